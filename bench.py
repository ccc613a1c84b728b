"""Benchmark of the relative-attention hot path on one MI355X.

A step is one prefill call (the whole forward: scores, relative bias, mask,
online softmax, PV, epilogue) of the full-attention layer with the length
log-scale (B=2, T=32768, Hq=16, Hkv=2, D=128, d_r=128, rel_extent=1024,
causal, s = 1.25, bf16), the largest prefill that fits one GPU, on inputs
already resident in HBM.  Its algorithmic TFLOP/s is the headline `value`,
with the kernel's fraction of the bf16 MFMA peak in `roofline`.

The same line carries one object per other named workload, each with its own
roofline and the fp64 CPU oracle timed on a bounded sample of it:
  * tiny_fp32       B=1 T=256 Hq=4 Hkv=1 d_r=32 E=64, fp32 (launch-bound)
  * swa_prefill_8k  B=1 T=8192 Hq=16 Hkv=2 d_r=128 E=1024 W=1024
  * decode_64x8k    64 sequences x 1 token over 8192 keys (KV GB/s vs HBM)
  * decode_1x1m_log 1 sequence x 1 token over 2^20 keys, s = 5/3
and the rows the library adds beside the forward (paged and MXFP8 decode,
extend over a paged cache in bf16 and in MXFP8, the attention prologue, the
backward).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only NAME[,NAME...]]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for
           scaling the HBM byte counters FETCH_SIZE / WRITE_SIZE)
       python bench.py --hbm-ceiling   (plain copy and sum rates: a yardstick)
       python bench.py --ceilings   (plain MFMA, exp, LDS-read rates and the
           shader clock: yardsticks beside the published peaks)
       python bench.py --traffic-from FETCH_CSV WRITE_CSV --kernel-key KEY
                       --kernel-match SUBSTR[,SUBSTR...] --src FILE[,FILE...]
           (turn two rocprofv3 --pmc counter CSVs into the per-launch HBM
           bytes of profiles/traffic.json; see `traffic_from_counters`)
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector, published (the fp32 path runs fp32 MFMA / VALU)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
METRIC = "relative-attention prefill TFLOP/s + decode KV GB/s (% of MI355X peak)"
HEADLINE = "full_prefill_32k_log"
PREFILL_WORKLOADS = ["tiny_fp32", "swa_prefill_8k", "full_prefill_32k_log"]
DECODE_WORKLOADS = ["decode_64x8k", "decode_1x1m_log"]
EXTRA = ["decode_paged", "decode_mx", "extend", "extend_mx", "prologue", "backward"]
EXTEND_WORKLOAD = "extend_4x1k_8k_paged"
PAGED_DECODE_WORKLOAD = "decode_paged_64x8k"
PROLOGUE_WORKLOAD = "prologue_8k"
BACKWARD_WORKLOAD = "swa_backward_8k"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


# ----------------------------------------------------------------------------
# algorithmic work


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


def decode_bytes_mx(B: int, L: int, Hq: int, Hkv: int, D: int, d_r: int, E: int, W: int) -> int:
    """Algorithmic bytes of one decode call over MXFP8 caches: per visible key
    and kv head the K and V codes (D bytes each) and scales (D/32 bytes
    each); q, r and out per sequence (bf16) and P once, as for bf16."""
    vis = min(L, W) if W > 0 else L
    kv = B * vis * Hkv * 2 * (D + D // 32)
    per_seq = B * (Hq * D * 2 + Hq * d_r * 2 + Hq * D * 2)
    return kv + per_seq + E * d_r * 2


def prologue_bytes(N: int, B: int, Hq: int, Hkv: int, D: int, W: int, state: bool, elem: int = 2) -> int:
    """Algorithmic bytes of one prologue call: every q, k and v row read once
    and written once (q_out, the two caches), the filter and norm weights, and
    the states (read if given, always written)."""
    rows = 2 * N * (Hq + 2 * Hkv) * D * elem
    weights = (2 * Hkv * D * W + 2 * D) * elem
    st = B * 2 * 3 * Hkv * D * elem
    return rows + weights + st * (2 if state else 1)


# ----------------------------------------------------------------------------
# counters


def src_hash(*names):
    """Hash of kernel sources: a counter reading is used only while the source
    it was taken on is unchanged."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "transformer_attention_query_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


PREFILL_SRC = ("prefill.hip", "device_common.hpp", "mx_common.hpp")
DECODE_SRC = ("decode.hip", "device_common.hpp", "mx_common.hpp")


def traffic(key: str, src):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        data = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("src_hash") != src_hash(*src):
        return None
    return ent.get("bytes_per_launch")


def _counter_means(path: str, counter: str):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3
    counter-collection CSV."""
    acc = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_from_counters(fetch_csv: str, write_csv: str, key: str, matches, src, calib=None):
    """HBM bytes per launch of the kernels whose names contain one of `matches`
    (summed over them: e.g. a split kernel and its merge make one call).

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; each is scaled by
    the factor a plain device copy of known size gives for the same counter
    (`_calibration` in traffic.json: bytes = scale * KiB * 1024)."""
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    cal = data.get("_calibration") if calib is None else calib
    if not cal:
        raise SystemExit("no _calibration in traffic.json: run the copy calibration first")
    F = _counter_means(fetch_csv, "FETCH_SIZE")
    W = _counter_means(write_csv, "WRITE_SIZE")
    fetch = write = 0.0
    per = {}
    for m in matches:
        names = [k for k in F if m in k]
        if len(names) != 1:
            raise SystemExit(f"kernel match {m!r} selects {names}")
        n = names[0]
        f = F[n] * 1024 * cal["fetch_scale"]
        w = W.get(n, 0.0) * 1024 * cal["write_scale"]
        per[m] = {"fetch_bytes": int(f), "write_bytes": int(w)}
        fetch += f
        write += w
    data[key] = {"src_hash": src_hash(*src), "fetch_bytes": int(fetch), "write_bytes": int(write),
                 "bytes_per_launch": int(fetch + write), "kernels": per}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps({key: data[key]}))


def calibration_from_counters(fetch_csv: str, write_csv: str, nbytes: int = 1 << 30):
    """Counter scale factors from the plain copy kernel of `copy_calibration`."""
    F = _counter_means(fetch_csv, "FETCH_SIZE")
    W = _counter_means(write_csv, "WRITE_SIZE")
    fk = max(F.values())
    wk = max(W.values())
    cal = {"copy_bytes": nbytes, "FETCH_SIZE_KiB": fk, "WRITE_SIZE_KiB": wk,
           "fetch_scale": nbytes / (fk * 1024), "write_scale": nbytes / (wk * 1024)}
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data["_calibration"] = cal
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(cal))


# ----------------------------------------------------------------------------
# timing


def _time_launches(fn, steps: int, warmup: int, stream):
    """Run fn(i) warmup times, then `steps` times between synchronisations,
    with a HIP event pair on the launch stream around every launch.
    Returns (total ms over the steps, list of per-launch ms)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
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


def _time_calls(fn, steps: int, warmup: int, stream):
    """Short library calls (decode: a split kernel and a merge, ~0.1-0.2 ms):
    the timed region is `steps` calls back to back between one pair of HIP
    events on the launch stream, so no event sits between the kernels of
    consecutive calls (an event pair around every call adds ~2-5 us of
    event processing to each 100-200 us call).  Returns (ms per call over
    the timed region, per-call ms from a second pass with an event pair
    around every call, for the spread)."""
    ms = _time_batch(fn, steps, warmup, stream)
    _, per = _time_launches(fn, steps, 1, stream)
    return ms, per


def _stats(per):
    s = sorted(per)
    return {"avg_launch_us": round(sum(s) / len(s) * 1e3, 2), "median_us": round(s[len(s) // 2] * 1e3, 2),
            "min_us": round(s[0] * 1e3, 2), "max_us": round(s[-1] * 1e3, 2)}


def _roofline(bound, kernel, achieved, peak, unit, tr, per, avg_ms=None):
    r = {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": tr}
    if avg_ms is None:
        r.update(_stats(per))
    else:  # timed region of back-to-back calls; the spread from per-call events
        r["avg_launch_us"] = round(avg_ms * 1e3, 2)
        r["timing"] = "one HIP event pair around the timed calls"
        r.update({"per_call_events_" + k: v for k, v in _stats(per).items()})
    return r


# ----------------------------------------------------------------------------
# the CPU oracle as a reported baseline


def _host():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def oracle_prefill_time(w, x, target_s: float):
    """The fp64 oracle, as it stands, on evenly spaced query rows of a prefill
    workload (all rows when they fit the time target)."""
    import torch
    import oracle
    T = w.T
    stride_rows = lambda n: list(range(T - 1, -1, -max(1, T // n)))[:n]  # noqa: E731
    run = lambda rows: oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W,  # noqa: E731
                                      w.log_scale, rows=rows)
    run(stride_rows(4))
    t = time.perf_counter()
    run(stride_rows(16))
    per_row = (time.perf_counter() - t) / 16
    n = int(max(16, min(T, target_s / max(per_row, 1e-6))))
    rows = stride_rows(n)
    reps = 0
    t = time.perf_counter()
    while True:  # a workload the oracle finishes in well under a second is repeated
        run(rows)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min(1.0, target_s) or len(rows) < T:
            break
    dt /= reps
    flops, _, _ = prefill_work(T, w.Hq, w.D, w.d_r, w.E, w.W, rows=rows)
    flops *= w.B
    cpus, model = _host()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(), "host_cpus": cpus,
            "cpu_model": model, "kind": "oracle", "wall_s": round(dt, 2),
            "sample": f"{len(rows)} of {T} query rows (evenly spaced from the last; every head and sequence) "
                      f"of {w.name}, fp64 torch-CPU oracle"}


def oracle_decode_time(w, x, target_s: float):
    """The fp64 oracle, as it stands, on the first sequences of a decode
    workload (all of them when they fit the time target)."""
    import torch
    import oracle
    sub = lambda n: {k: (t[:n] if k in ("q", "k", "v", "r") else t) for k, t in x.items()}  # noqa: E731
    run = lambda y: oracle.decode(y["q"], y["k"], y["v"], y["r"], y["P"], w.alpha, w.E, w.W, w.log_scale)  # noqa: E731
    t = time.perf_counter()
    run(sub(1))
    per_seq = time.perf_counter() - t
    n = int(max(1, min(w.B, target_s / max(per_seq, 1e-6))))
    t = time.perf_counter()
    if n > 1 or w.B > 1:
        run(sub(n))
        dt = time.perf_counter() - t
    else:
        dt = per_seq
    nbytes, _ = decode_bytes(n, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    cpus, model = _host()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": torch.get_num_threads(), "host_cpus": cpus,
            "cpu_model": model, "kind": "oracle", "wall_s": round(dt, 2),
            "sample": f"{n} of {w.B} sequences (all {w.Hq} heads, all {w.T} keys) of {w.name}, "
                      f"fp64 torch-CPU oracle"}


# ----------------------------------------------------------------------------
# workloads


def bench_prefill(name: str, steps: int, warmup: int, cpu: bool):
    """One prefill workload: per-launch HIP events on the launch stream.  The
    8K workload's inputs (76 MB) would stay in the 256 MB MALL between
    launches, so it rotates over four copies (304 MB); the 32K workload's
    inputs (576 MB) exceed the MALL by themselves."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[name]
    xc = tinputs.make_inputs(w, seed=0)
    x = {n: t.cuda() for n, t in xc.items()}
    n_copies = 4 if name == "swa_prefill_8k" else 1
    sets = [x] + [{n: t.clone() for n, t in x.items()} for _ in range(n_copies - 1)]
    out = torch.empty_like(x["q"])
    lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        y = sets[i % n_copies]
        ra.prefill(y["q"], y["k"], y["v"], y["r"], y["P_cols"], w.alpha, w.E, w.W, w.log_scale, out=out, lse=lse)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    flops, pairs, rel = prefill_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W)
    flops *= w.B
    ms_step = total_ms / steps
    kernel_ms = sum(per) / len(per)
    bf16 = w.dtype == "bf16"
    G = w.Hq // w.Hkv
    kernel = "prefill_dma_kernel" if bf16 and G % 8 == 0 else f"prefill_kernel<{'__bf16, 8' if bf16 else 'float, 2'}>"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    obj = {"workload": w.name, "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
           "ms_per_step": round(ms_step, 5), "dtype": w.dtype,
           "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "d_r": w.d_r,
                      "rel_extent": w.E, "window": w.W, "log_scale": w.log_scale, "alpha": "1/sqrt(128)",
                      "algorithmic_flops": flops, "visible_pairs": pairs * w.B, "rel_entries": rel * w.B,
                      "input_copies_rotated": n_copies},
           "roofline": _roofline("mfma", kernel, achieved, peak, "TFLOP/s",
                                 traffic(f"{kernel.split('<')[0]}@{w.name}", PREFILL_SRC), per)}
    if not bf16:
        obj["roofline"]["note"] = ("fp32 path against the fp32 vector peak; launch-bound at this size "
                                   "(parity workload)")
    print(f"# prefill {w.name}: {ms_step * 1e3:.1f} us/step, kernel {kernel_ms * 1e3:.1f} us "
          f"({achieved:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    del sets, x, out, lse
    torch.cuda.empty_cache()
    if cpu:
        obj["cpu_baseline"] = oracle_prefill_time(w, xc, 15.0 if name == HEADLINE else 8.0)
        print(f"# oracle {w.name}: {obj['cpu_baseline']['sample']}, {obj['cpu_baseline']['wall_s']} s",
              file=sys.stderr, flush=True)
    return obj


def bench_decode(name: str, steps: int, warmup: int, cpu: bool):
    """One decode workload (the split kernel and the merge, per call).  Two
    copies of the cache, used alternately: each launch reads at least 512 MiB,
    so the copy it reads was last touched two launches ago, beyond the 256 MB
    MALL and the L2s."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[name]
    xc = tinputs.make_inputs(w, seed=0)
    x = {n: t.cuda() for n, t in xc.items()}
    k2 = [x["k"], x["k"].clone()]
    v2 = [x["v"], x["v"].clone()]
    ns, ws_bytes = ra.decode_plan(w.B, w.T, w.Hq, w.Hkv, w.D, w.num_splits, w.W, w.E)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        ra.decode(x["q"], k2[i % 2], v2[i % 2], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale,
                  num_splits=ns, workspace=ws)

    ms_step, per = _time_calls(step, steps, warmup, stream)
    nbytes, kv = decode_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    kernel_ms = ms_step
    kgbps = nbytes / (kernel_ms * 1e-3) / 1e9
    obj = {"workload": w.name, "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
           "ms_per_step": round(ms_step, 5), "num_splits": ns, "algorithmic_bytes": nbytes, "dtype": "bf16",
           "config": {"workload": w.name, "B": w.B, "L": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "d_r": w.d_r,
                      "rel_extent": w.E, "window": w.W, "log_scale": w.log_scale, "kv_copies_rotated": 2},
           "roofline": _roofline("hbm", "decode_split_kernel+merge", kgbps, PEAK_HBM_GBPS, "GB/s",
                                 traffic(f"decode_split_kernel@{w.name}", DECODE_SRC), per, kernel_ms)}
    print(f"# decode {w.name}: {ms_step * 1e3:.1f} us/step, call {kernel_ms * 1e3:.1f} us ({ns} splits, "
          f"{kgbps:.0f} GB/s)", file=sys.stderr, flush=True)
    del x, k2, v2, ws
    torch.cuda.empty_cache()
    if cpu:
        obj["cpu_baseline"] = oracle_decode_time(w, xc, 8.0)
        print(f"# oracle {w.name}: {obj['cpu_baseline']['sample']}, {obj['cpu_baseline']['wall_s']} s",
              file=sys.stderr, flush=True)
    return obj


def bench_decode_mx(steps: int, warmup: int):
    """decode_64x8k over MXFP8 caches (quantised once from the bf16 ones)."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS["decode_64x8k"]
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

    ms, per = _time_calls(step, steps, warmup, stream)
    nbytes = decode_bytes_mx(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    k = nbytes / (ms * 1e-3) / 1e9
    print(f"# decode {w.name} (MXFP8 K/V): {ms * 1e3:.1f} us/step ({ns} splits)", file=sys.stderr, flush=True)
    return {"workload": w.name + " (MXFP8 K/V)", "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 5), "num_splits": ns, "algorithmic_bytes": nbytes,
            "dtype": "mxfp8 K/V, bf16 q/out",
            "roofline": _roofline("hbm", "decode_split_kernel (MXFP8)+merge", k, PEAK_HBM_GBPS, "GB/s",
                                  traffic("decode_split_kernel_mx@decode_64x8k", DECODE_SRC), per, ms)}


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

    ms, per = _time_calls(step, steps, warmup, stream)
    nbytes, _ = decode_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    k = nbytes / (ms * 1e-3) / 1e9
    print(f"# decode {w.name}: {ms * 1e3:.1f} us/step ({ns} splits)", file=sys.stderr, flush=True)
    return {"workload": w.name, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 5), "num_splits": ns, "algorithmic_bytes": nbytes,
            "roofline": _roofline("hbm", "decode_split_kernel (paged)+merge", k, PEAK_HBM_GBPS, "GB/s",
                                  traffic(f"decode_split_kernel_paged@{w.name}", DECODE_SRC), per, ms)}


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
    flops *= w.B
    ms = total_ms / steps
    ach = flops / (sum(per) / len(per) * 1e-3) / 1e12
    print(f"# extend {w.name}: {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    return {"workload": w.name, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms, 5), "algorithmic_flops": flops,
            "config": {"B": w.B, "kv_len": w.T, "new_rows": w.n_new, "page_size": w.page_size, "Hq": w.Hq,
                       "Hkv": w.Hkv, "d_r": w.d_r, "rel_extent": w.E, "window": w.W},
            "roofline": _roofline("mfma", "prefill_dma_kernel (extend)", ach, PEAK_BF16_TFLOPS, "TFLOP/s",
                                  traffic(f"prefill_dma_kernel_extend@{w.name}", PREFILL_SRC), per)}


def bench_extend_mx(steps: int, warmup: int):
    """The extend workload over MXFP8 caches (quantised once from the bf16 pages)."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[EXTEND_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    paged = w.page_size > 0
    kc, ks = ra.mx_quantize(x["k_pages"] if paged else x["k"])
    vc, vs = ra.mx_quantize(x["v_pages"] if paged else x["v"])
    bt = x["block_table"] if paged else None
    stream = torch.cuda.current_stream()

    def step(_i):
        ra.extend_mx(x["q"], kc, ks, vc, vs, x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale, x["q_start"],
                     x["kv_len"], w.n_new, block_table=bt)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    flops, _, _ = prefill_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W, rows=range(w.T - w.n_new, w.T))
    flops *= w.B
    ms = total_ms / steps
    ach = flops / (sum(per) / len(per) * 1e-3) / 1e12
    print(f"# extend {w.name} (MXFP8 K/V): {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    return {"workload": w.name + "_mx", "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms, 5), "algorithmic_flops": flops, "kv_format": "MXFP8 (E4M3 + E8M0 per 32)",
            "config": {"B": w.B, "kv_len": w.T, "new_rows": w.n_new, "page_size": w.page_size, "Hq": w.Hq,
                       "Hkv": w.Hkv, "d_r": w.d_r, "rel_extent": w.E, "window": w.W},
            "roofline": _roofline("mfma", "prefill_kernel (extend, MXFP8)", ach, PEAK_BF16_TFLOPS, "TFLOP/s",
                                  traffic(f"prefill_kernel_extend_mx@{w.name}", PREFILL_SRC), per),
            "note": "scores on the fp8 MFMA, P.V and r.P on bf16; priced against the bf16 peak"}


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

    total_ms, per = _time_launches(step, steps, warmup, stream)
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
    ms = total_ms / steps
    gk = nbytes / (kernel_ms * 1e-3) / 1e9
    print(f"# prologue {w.name}: {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    roof = _roofline("hbm", "prologue_kernel", gk, PEAK_HBM_GBPS, "GB/s",
                     traffic(f"prologue_kernel@{w.name}", ("prologue.hip", "device_common.hpp", "mx_common.hpp")),
                     per)
    roof["avg_launch_us"] = round(kernel_ms * 1e3, 2)
    roof["timing"] = "avg over back-to-back launches through the C ABI; min/max/median from per-call events"
    return {"workload": w.name, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 5), "algorithmic_bytes": nbytes,
            "config": {"B": w.B, "tokens": N, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "conv_width": 4,
                       "page_size": w.page_size},
            "roofline": roof}


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
    ms = total_ms / steps
    ach = flops / (sum(per) / len(per) * 1e-3) / 1e12
    print(f"# backward {w.name}: {ms * 1e3:.1f} us/step ({ns} head splits)", file=sys.stderr, flush=True)
    return {"workload": w.name, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(ms, 5), "algorithmic_flops": flops, "head_splits": ns,
            "config": {"B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "d_r": w.d_r, "rel_extent": w.E,
                       "window": w.W, "log_scale": w.log_scale},
            "roofline": _roofline("mfma", "bwd_dq_kernel+bwd_dkdv_kernel (+delta, reduce)", ach, PEAK_BF16_TFLOPS,
                                  "TFLOP/s", traffic(f"backward@{w.name}", ("backward.hip", "device_common.hpp")),
                                  per)}


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


def hbm_ceiling(nbytes: int = 4 << 30, reps: int = 10):
    """What plain streaming reaches on this GPU, as a yardstick for the decode
    fractions: a read-only kernel (libceilings.so, built beside the library:
    16-byte loads, four in flight per thread, grid-stride) over nbytes at
    several grid sizes, and torch's device-to-device copy (reads and writes
    nbytes); HIP events around `reps` back-to-back runs after one warm-up."""
    import ctypes
    import torch
    from transformer_attention_query_amd import build as _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.hbm_read_probe.restype = ctypes.c_int
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    out = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    for blocks in (2048, 8192, 16384, 32768, 65536):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")

        def read():
            rc = lib.hbm_read_probe(src.data_ptr(), nbytes, blocks, sink.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"hbm_read_probe returned {rc}")
        ms = timed(read)
        out[f"read_{blocks}x256"] = {"bytes": nbytes, "us": round(ms * 1e3, 1),
                                     "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    ms = timed(lambda: dst.copy_(src))
    out["torch_copy"] = {"bytes": 2 * nbytes, "us": round(ms * 1e3, 1),
                         "GB_per_s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"hbm_ceiling": out, "peak_GB_per_s": PEAK_HBM_GBPS}), flush=True)


def compute_ceilings():
    """What plain code of each kind reaches on this GPU (libceilings.so):
    back-to-back bf16 32x32x16 MFMAs with four independent accumulators per
    wave at 1, 2 and 4 waves per SIMD; independent v_exp_f32 chains; 16-byte
    LDS reads; and the shader clock against the 100 MHz real-time counter.
    HIP events around one launch after a warm-up launch."""
    import ctypes
    import torch
    from transformer_attention_query_amd import build as _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    lib.ceiling_threads.argtypes = [ctypes.c_int]
    lib.ceiling_threads.restype = ctypes.c_size_t
    lib.compute_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.compute_probe.restype = ctypes.c_int
    lib.clock_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.clock_probe.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e-3  # seconds

    def probe(kind, blocks, iters):
        sink = torch.empty(int(lib.ceiling_threads(blocks)), dtype=torch.int32, device="cuda")

        def run():
            rc = lib.compute_probe(kind, blocks, iters, sink.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"compute_probe({kind}) returned {rc}")
        return timed(run)

    out = {"compute_units": n_cu}
    blocks = 256
    sink = torch.empty(int(lib.ceiling_threads(blocks)), dtype=torch.int32, device="cuda")
    ticks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    rc = lib.clock_probe(blocks, 200000, ticks.data_ptr(), sink.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    if rc != 0:
        raise RuntimeError(f"clock_probe returned {rc}")
    t = ticks.view(blocks, 2).double().cpu()
    mhz = float((t[:, 0] / t[:, 1]).median()) * 100.0
    out["shader_clock_MHz"] = round(mhz, 1)
    mfma = {}
    for waves_per_simd in (1, 2, 4):
        blocks = n_cu * waves_per_simd
        iters = 20000
        sec = probe(0, blocks, iters)
        flops = blocks * 4 * iters * 4 * 32768
        tf = flops / sec / 1e12
        mfma[f"{waves_per_simd}_wave_per_simd"] = {"TFLOP_per_s": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    out["mfma_bf16_32x32x16"] = mfma
    blocks, iters = 4 * n_cu, 5000
    sec = probe(1, blocks, iters)
    n_exp = blocks * 256 * iters * 8
    out["v_exp_f32"] = {"G_per_s": round(n_exp / sec / 1e9, 1),
                        "per_clock_per_cu": round(n_exp / sec / (mhz * 1e6) / n_cu, 1)}
    for kind, name in ((2, "lds_read_b128_consecutive"), (3, "lds_read_b128_fragment_rows")):
        blocks, iters = 4 * n_cu, 5000
        sec = probe(kind, blocks, iters)
        nbytes = blocks * 256 * iters * 4 * 16
        out[name] = {"TB_per_s": round(nbytes / sec / 1e12, 2),
                     "bytes_per_clock_per_cu": round(nbytes / sec / (mhz * 1e6) / n_cu, 1)}
    print(json.dumps({"ceilings": out, "peak_bf16_TFLOP_per_s": PEAK_BF16_TFLOPS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma-separated workloads / extra sections to run")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--hbm-ceiling", action="store_true", help="time a plain copy and a plain sum (yardstick)")
    ap.add_argument("--ceilings", action="store_true", help="plain MFMA, exp and LDS rates and the shader clock")
    ap.add_argument("--calibration-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--kernel-key")
    ap.add_argument("--kernel-match")
    ap.add_argument("--src")
    args = ap.parse_args()
    if args.calibration_from:
        calibration_from_counters(*args.calibration_from)
        return
    if args.traffic_from:
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.kernel_key,
                              args.kernel_match.split(","), args.src.split(","))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the relative-attention kernels run on a single MI355X "
              "and the library has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
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
    if args.hbm_ceiling:
        hbm_ceiling()
        return
    if args.ceilings:
        compute_ceilings()
        return

    only = set(s for s in args.only.split(",") if s)
    want = lambda n: not only or n in only  # noqa: E731
    cpu = not args.no_cpu_baseline

    line = {"metric": METRIC}
    objs = {}
    for name in PREFILL_WORKLOADS:
        if want(name):
            objs[name] = bench_prefill(name, args.steps, args.warmup, cpu)
    for name in DECODE_WORKLOADS:
        if want(name):
            objs[name] = bench_decode(name, args.steps, args.warmup, cpu)
    if HEADLINE in objs:
        h = objs.pop(HEADLINE)
        line.update({"value": h["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                     "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True,
                     "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                     "config": h["config"], "roofline": h["roofline"]})
        if "cpu_baseline" in h:
            line["cpu_baseline"] = h["cpu_baseline"]
    else:
        line.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "note": "headline not run (--only)"})
    line.update(objs)
    extras = {"decode_paged": bench_decode_paged, "decode_mx": bench_decode_mx, "extend": bench_extend,
              "extend_mx": bench_extend_mx, "prologue": bench_prologue, "backward": bench_backward}
    for key in EXTRA:
        if want(key):
            line[key] = extras[key](args.steps, args.warmup)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
