"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunked prefill of the at-scale workload (B=1, H=HV=96,
T=8192, K=V=128, zero fp32 initial state) followed by one decode step of the
B=256 decode workload (H=HV=12, bf16 state pool [1024,12,128,128], 1/8 of the
rows inactive).  Inputs are synthetic (seeded, generated on the host, copied
to HBM before timing).  The prefill's 1.2 GB of traffic evicts the decode
pool's slots from the 256 MB last-level cache between decode calls, so the
decode runs cache-cold.

Prints one JSON line:
  value        prefill tokens/s (T / mean prefill call time by HIP events)
  roofline     the prefill entry point -- on this workload the split form's
               overlapped schedule: one chunk-kernel launch, the carry
               beside its later rows on the library's second stream, joined
               back into the launch stream; the call timed by HIP events on
               the launch stream -- against the HBM roofline: algorithmic
               bytes per call / mean call time.  traffic is the measured HBM bytes per
               call from the committed rocprofv3 counter summary when that
               was taken on the current kernel source, else null
  prefill, decode  event statistics (mean, p10, median, p90), the device
               kernel durations (no launch gaps) from the committed
               rocprofv3 kernel trace of these steps when it was taken on
               the current kernel sources, and the same calls after a 1 GiB
               cache-flushing read
  configs      the other workloads (the small prefills, the varlen GQA
               batch, decode at B = 1, 8, 32, 256), each after a cache
               flush, with its algorithmic bytes and roofline fractions
  handoff,     the prefill-to-decode handoff (256 x 12 fp32 states into the
  packed_decode  pool) and the packed-input decode (B=256, H=12), each timed
               with a prefill before every launch, so they too meet the
               caches the way they would in serving
  prefill_partitions  mean call time of the split and the fused prefill
               partitions (on this workload also the split form's
               sequential schedule) on this workload, on the 16-sequence varlen GQA
               batch (512 units) and on B=16 H=HV=64 T=2048 (1024 units),
               with the one kda_chunk_prefill picks ("auto")
  backward     the prefill's backward on this workload (float32 ALU roofline)
  measured_ceilings  copy / read / write bandwidth and a bf16 GEMM on this
               box, beside the vendor peaks
  cpu_baseline the fp64 oracle (token-by-token form) on a bounded sample of
               the same prefill workload, on all of this host's cores
Only --gpus 1 is supported: the library runs on one GPU.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s @H=96,T=8192 (% MFMA peak); decode state GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 MFMA

K = V = 128
C = 64


def prefill_alg_bytes(T_tot, H, HV, N, has_init):
    """Inputs read once, outputs written once: q,k (bf16), v (bf16), g (fp32),
    beta (bf16), o (bf16), initial state (fp32, when given), final state (fp32)."""
    per_tok = H * 2 * K * 2 + HV * (V * 2 + K * 4 + 2 + V * 2)
    states = N * HV * K * V * 4 * ((1 if has_init else 0) + 1)
    return T_tot * per_tok + states


def prefill_alg_flops(T_tot, HV):
    """Chunk form at C=64 with triangles exploited, per token and value head:
    6KV (W S, Qg S, Kg^T Vnew) + (C-1)K (L) + 2(C+1)K (Aqk, W)
    + 2(C+1)V (U, Aqk Vnew) + C^2/3 (solve)."""
    per = 6 * K * V + (C - 1) * K + 2 * (C + 1) * K + 2 * (C + 1) * V + C * C / 3
    return T_tot * HV * per


FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector (and fp32 MFMA)


def backward_alg_bytes(T_tot, H, HV, N, has_init, has_dht):
    """Backward inputs read once (q, k, v, beta, d_out bf16; g fp32; initial
    state and final-state gradient fp32) and the gradients written once in
    their inputs' dtypes (dq, dk, dv, dbeta bf16; dg, d_initial_state
    fp32)."""
    per_tok = H * 2 * K * 2 + HV * (V * 2 + K * 4 + 2 + V * 2)          # inputs
    per_tok += H * 2 * K * 2 + HV * (V * 2 + K * 4 + 2)                 # gradients
    states = N * HV * K * V * 4 * ((1 if has_init else 0) + (1 if has_dht else 0) + 1)
    return T_tot * per_tok + states


def backward_alg_flops(n_chunk_heads):
    """Per (64-token chunk, value head), multiply-adds counted as 2 flops,
    triangles exploited (P = C(C+1)/2 lower-triangle pairs incl. the
    diagonal, M = C*K*V):
      recompute: P, Aqk, W, U over the triangle: 4 * 2 P K; solve 2 C^3/6
      forward carry: W S, Kg^T Vnew: 2 * 2M
      reverse carry: Kg dS', Qg^T dO, W^T dVnew: 3 * 2M; Aqk^T dO: 2 P V
      gradients: dO S^T, Vnew dS'^T, dVnew S^T: 3 * 2M; dAqk, dA (two
      terms), dv, dE: 5 * 2 P K; dT T^T and T^T X: 2 C^3/3 + 2 C^3/6;
      the four gated sums: 4 * 2 P K; dgamma 2 K V."""
    P = C * (C + 1) // 2
    M = C * K * V
    per = (4 * 2 * P * K + 2 * C ** 3 / 6
           + 2 * 2 * M
           + 3 * 2 * M + 2 * P * V
           + 3 * 2 * M + 5 * 2 * P * K + 2 * C ** 3 / 3 + 2 * C ** 3 / 6 + 4 * 2 * P * K + 2 * K * V)
    return n_chunk_heads * per


def decode_alg_bytes(B_act, B_inact, H, HV):
    """Active rows read and write their bf16 state slot and read q,k,v,g,beta
    and write o; inactive rows write zero o; plus the int32 indices."""
    per = 2 * K * V * 2 + 2 * K * 2 * H / HV + V * 2 + K * 4 + 2 + V * 2
    return B_act * HV * per + 4 * (B_act + B_inact) + B_inact * HV * V * 2


def source_hash(name):
    """Hash of a kernel source's code with comments and blank lines removed,
    so that a comment edit does not invalidate a counter record."""
    path = os.path.join(ROOT, "kda_gated_delta_amd", "csrc", name)
    text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    lines = [re.sub(r"//.*", "", line).rstrip() for line in text.splitlines()]
    code = "\n".join(line for line in lines if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


KTRACE_PATH = os.path.join(ROOT, "profiles", "kernel_trace_h96_t8192.json")


def flag_room(B, T, HV, nseq=0):
    """Bytes of ready flags and unit status words at the end of the
    prefill's full workspace (see kda_chunk_prefill_workspace_size in
    include/kda.h)."""
    nslots = (B * T) // C + (nseq or B) + 1
    return ((nslots + (nseq or B)) * HV * 4 + 255) // 256 * 256


def kernel_trace_summary(stats_csv, out_path):
    """Device durations from a rocprofv3 --kernel-trace --stats run of
    `bench.py --only-steps` (run_kernel_stats.csv and, beside it,
    run_kernel_trace.csv), recorded with the hashes of the kernel sources
    they were measured on: each kernel's average, and the prefill call's
    device span (first kernel start to last kernel end; its kernels overlap
    in the overlapped split schedule, so their durations do not add up)."""
    import csv
    rec = {"workload": "prefill B=1 H=HV=96 T=8192 then decode B=256 H=HV=12, back-to-back steps",
           "source": "rocprofv3 --kernel-trace --stats (kernel start to end on the device)",
           "prefill_code_sha256_16": source_hash("prefill.hip"),
           "decode_code_sha256_16": source_hash("decode.hip"), "kernels_us": {}}
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            name = row["Name"]
            m = re.search(r"(intra_kernel|inter_kernel|clear_flags_kernel|decode_kernel)(<[^(]*>)?", name)
            if m and ("decode" not in m.group(1) or "SplitInputs" in name):
                key = m.group(1) + (m.group(2) or "").replace("(anonymous namespace)::", "")
                rec["kernels_us"][key] = float(row["AverageNs"]) / 1e3
    trace_csv = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace("kernel_stats", "kernel_trace"))
    spans = []
    with open(trace_csv) as f:
        rows = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in csv.DictReader(f)))
    call = None
    for t0, t1, name in rows:
        if "intra_kernel" in name or "inter_kernel" in name or "clear_flags_kernel" in name:
            call = [t0, t1] if call is None else [min(call[0], t0), max(call[1], t1)]
        elif call is not None:             # the decode (or anything else) ends the prefill call
            spans.append((call[1] - call[0]) / 1e3)
            call = None
    if call is not None:
        spans.append((call[1] - call[0]) / 1e3)
    rec["prefill_call_span_us"] = sum(spans) / len(spans) if spans else None
    rec["prefill_calls"] = len(spans)
    with open(out_path, "w") as fo:
        json.dump(rec, fo, indent=1)
        fo.write("\n")
    print(json.dumps(rec), flush=True)


def kernel_trace_from_profiles():
    """The committed rocprofv3 kernel averages, if taken on the current
    kernel sources (else None)."""
    if not os.path.exists(KTRACE_PATH):
        return None
    try:
        rec = json.load(open(KTRACE_PATH))
    except ValueError:
        return None
    if rec.get("prefill_code_sha256_16") != source_hash("prefill.hip") or \
            rec.get("decode_code_sha256_16") != source_hash("decode.hip"):
        return None
    return rec


def traffic_from_profiles():
    """Per-launch HBM bytes of the prefill kernel from the committed counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "prefill_h96_t8192_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    if rec.get("prefill_code_sha256_16") != source_hash("prefill.hip"):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_cpu_s):
    """Time the fp64 recurrent oracle on a bounded sample of the prefill
    workload -- every value head over the first tokens -- on all of this
    host's cores (one process per head, at most 16), sized from a pilot so
    that the sample costs about `target_cpu_s` seconds of CPU time.
    Reported as tokens/s of the sample (all heads of each token)."""
    import multiprocessing as mp
    from oracle.parallel import _task, default_workers
    T = inp.q.shape[1]
    HV = inp.v.shape[2]
    H = inp.q.shape[2]
    grp = HV // H
    workers = default_workers()

    def tasks(n):
        out = []
        for h in range(H):
            hv = slice(h * grp, (h + 1) * grp)
            out.append((inp.q[:, :n, h:h + 1].float().numpy(), inp.k[:, :n, h:h + 1].float().numpy(),
                        inp.v[:, :n, hv].float().numpy(), inp.g[:, :n, hv].numpy(),
                        inp.beta[:, :n, hv].float().numpy(), inp.initial_state[:, hv].numpy()))
        return out

    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map(_task, tasks(8)[:workers], chunksize=1)          # start-up, untimed
        n = 256
        c0, t0 = time.process_time(), time.perf_counter()
        ts = tasks(n)
        pool.map(_task, ts, chunksize=1)
        pilot = time.perf_counter() - t0
        # cpu seconds of the pilot = wall x busy workers (the pool's time is not in this process)
        per_tok_cpu = pilot * min(workers, len(ts)) / n
        n = int(min(T, max(n, target_cpu_s / max(per_tok_cpu, 1e-9))))
        ts = tasks(n)
        t0 = time.perf_counter()
        pool.map(_task, ts, chunksize=1)
        wall = time.perf_counter() - t0
    return {
        "value": n / wall,
        "unit": "tokens/s",
        "cores": min(workers, len(ts)),
        "kind": "oracle",
        "sample": f"fp64 token-by-token oracle on the prefill workload's first {n} of {T} tokens, all {HV} "
                  f"value heads, one process per head on {min(workers, len(ts))} worker processes "
                  f"({wall:.1f} s wall); host reports {os.cpu_count()} cpus",
    }


def handoff_alg_bytes(n_act, n_states, HV):
    """Active states are read as fp32 and written as bf16; plus the int32
    indices."""
    return n_act * HV * K * V * (4 + 2) + 4 * n_states


def packed_decode_alg_bytes(n_act, n_inact, H):
    """Active rows read and write their bf16 state slot and read their packed
    q|k|v row, raw gate and raw beta and write o; inactive rows write zero
    o; plus A_log, dt_bias and the int32 indices."""
    per = 2 * K * V * 2 + 3 * K * 2 + K * 2 + 2 + V * 2
    return n_act * H * per + n_inact * H * V * 2 + H * 4 + H * K * 4 + 4 * (n_act + n_inact)


def copy_calibration(nbytes):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, out_path):
    """Per-launch HBM bytes of the prefill entry point from rocprofv3 counter
    collections (FETCH_SIZE and WRITE_SIZE, KiB per dispatch), each scaled by
    what the counter reads for a plain copy of copy_bytes bytes."""
    import csv

    def per_kernel(path, counter):
        sums = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                sums.setdefault(name, []).append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in sums.items()}

    def short(name):
        m = re.search(r"(intra_kernel|inter_kernel|clear_flags_kernel)(<[^(]*>)?", name)
        return m.group(1) + (m.group(2) or "") if m else None

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    cf = max(per_kernel(copy_fetch_csv, "FETCH_SIZE").values())
    cw = max(per_kernel(copy_write_csv, "WRITE_SIZE").values())
    kib = copy_bytes / 1024.0
    f_scale, w_scale = cf / kib, cw / kib
    rec = {
        "workload": "prefill B=1 H=HV=96 T=8192 K=V=128",
        "prefill_code_sha256_16": source_hash("prefill.hip"),
        "copy_bytes": copy_bytes,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "kernels": {},
    }
    # Every prefill kernel is dispatched once per call, so a call's traffic
    # is the sum of the per-dispatch averages.  The overlapped schedule's
    # repair launch (inter_kernel<16> beside inter_kernel<32>) redoes only
    # units whose carry gave up waiting, which a normal call has none of; a
    # counter run serialises the kernels, and should its carry run before
    # the chunk kernel there, the repair would redo every unit: it is left
    # out when the 32-column carry is present.
    overlapped = any(short(n) == "inter_kernel<32>" for n in f)
    total = 0.0
    for name in f:
        key = short(name)
        if key is None or name not in w or (overlapped and key == "inter_kernel<16>"):
            continue
        fb = f[name] / f_scale * 1024.0
        wb = w[name] / w_scale * 1024.0
        rec["kernels"][key] = {"fetch_bytes": fb, "write_bytes": wb}
        total += fb + wb
    if not rec["kernels"]:
        raise SystemExit("no prefill dispatches in the counter files")
    rec["hbm_bytes_per_launch"] = total
    with open(out_path, "w") as fo:
        json.dump(rec, fo, indent=1)
        fo.write("\n")
    print(json.dumps(rec), flush=True)


def measure_backward(torch, synth, kda, pin, inputs, stream, steps, warmup):
    """Mean call time of kda_chunk_backward on the prefill workload (random
    upstream gradients), with its float32 ALU roofline: gradients of
    sum(o * d_out) + sum(final_state * d_final_state)."""
    print("[bench] backward", file=sys.stderr, flush=True)
    q, k, v, g, beta, s0 = inputs
    B, T, H, _ = pin.q.shape
    HV = pin.v.shape[2]
    dev = q.device
    d_out, d_final = synth.upstream_grads(pin)
    d_out, d_final = d_out.to(dev), d_final.to(dev)
    bws = torch.empty(kda.backward_workspace_size(B, T, H, HV), dtype=torch.uint8, device=dev)
    evs = []
    for i in range(warmup + steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.chunk_backward(q, k, v, g, beta, s0, d_out, d_final, workspace=bws)
        e1.record(stream)
        if i >= warmup:
            evs.append((e0, e1))
    torch.cuda.synchronize()
    bw_us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
    n_ch = B * ((T + C - 1) // C) * HV
    bw_flops = backward_alg_flops(n_ch)
    bw_bytes = backward_alg_bytes(B * T, H, HV, B, s0 is not None, True)
    del bws, d_out, d_final
    return {
        "workload": f"B={B} H=HV={HV} T={T}, float32",
        "call_us_mean": bw_us,
        "calls": steps,
        "tokens_per_s": B * T / (bw_us * 1e-6),
        "alg_flops": bw_flops,
        "alg_bytes": bw_bytes,
        "roofline": {"bound": "alu", "achieved": bw_flops / (bw_us * 1e-6) / 1e12, "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": bw_flops / (bw_us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS},
        "hbm_frac": bw_bytes / (bw_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
    }


def time_events(torch, stream, fn, n, warmup, flush=None):
    """Per-call times (ms) of fn by HIP events recorded on the launch stream.
    With `flush` (a callable), it runs before every call, outside the events
    (a write of a buffer larger than the last-level cache)."""
    evs = []
    for i in range(warmup + n):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        if i >= warmup:
            evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def stats_us(ms):
    xs = sorted(ms)
    return {"mean": sum(xs) / len(xs) * 1e3, "p10": xs[len(xs) // 10] * 1e3, "median": xs[len(xs) // 2] * 1e3,
            "p90": xs[(9 * len(xs)) // 10] * 1e3, "n": len(xs)}


def measured_ceilings(torch, dev):
    """What the chip delivers to plain library kernels on this machine: 1 GiB
    device copy (read + write), read-only reduction, write-only fill, and a
    bf16 GEMM (hipBLASLt via torch.matmul), beside the vendor peaks."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    f = a.view(torch.float32)
    stream = torch.cuda.current_stream()

    def best(fn, reps=8):
        return min(time_events(torch, stream, fn, reps, 2)) * 1e-3

    out = {}
    t = best(lambda: b.copy_(a))
    out["copy_gbs"] = 2 * n / t / 1e9
    t = best(lambda: f.sum())
    out["read_gbs"] = n / t / 1e9
    t = best(lambda: b.fill_(3))
    out["write_gbs"] = n / t / 1e9
    del a, b, f
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    y = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    t = best(lambda: torch.matmul(x, y), reps=10)
    out["bf16_gemm_tflops"] = 2 * m ** 3 / t / 1e12
    del x, y
    out["vendor"] = {"hbm_gbs": HBM_PEAK_GBS, "bf16_fp16_mfma_tflops": F16_PEAK_TFLOPS,
                     "fp32_tflops": FP32_PEAK_TFLOPS}
    out["kernels"] = "torch copy_/sum/fill_ (1 GiB, best of 8) and torch.matmul bf16 8192^3 (hipBLASLt)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=8192)
    ap.add_argument("--H", type=int, default=96)
    ap.add_argument("--decode-B", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="CPU seconds of the oracle sample for cpu_baseline (0 = skip)")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the backward of the prefill workload (for profiling)")
    ap.add_argument("--only-steps", action="store_true",
                    help="time only the steps (prefill + decode); skip everything else (for profiler runs "
                         "that average per kernel name)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_JSON"),
                    help="only summarise a rocprofv3 kernel-trace stats file into the kernel-time record")
    ap.add_argument("--traffic-summary", nargs=6, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                           "COPY_WRITE_CSV", "COPY_BYTES", "OUT_JSON"),
                    help="only summarise rocprofv3 counter files into the traffic record")
    args = ap.parse_args()
    if args.trace_summary:
        kernel_trace_summary(args.trace_summary[0], args.trace_summary[1])
        return
    if args.traffic_summary:
        a = args.traffic_summary
        traffic_summary(a[0], a[1], a[2], a[3], int(a[4]), a[5])
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import kda_gated_delta_amd as kda

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    kda.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] generating inputs T={args.T} H={args.H}", file=sys.stderr, flush=True)
    pin = synth.config2(T=args.T, H=args.H)
    q, k, v, g, beta = (t.to(dev) for t in (pin.q, pin.k, pin.v, pin.g, pin.beta))
    s0 = pin.initial_state.to(dev)
    B, T, H, _ = pin.q.shape
    HV = pin.v.shape[2]
    o = torch.empty(B, T, HV, V, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(B, HV, K, V, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_size(B, T, H, HV), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if args.only_backward:
        torch.cuda.synchronize()
        bw = measure_backward(torch, synth, kda, pin, (q, k, v, g, beta, s0), stream, args.steps, args.warmup)
        print(json.dumps({"backward": bw}), flush=True)
        return

    din = synth.decode_config(args.decode_B)
    dq, dk, dv, dg, db = (t.to(dev) for t in (din.q, din.k, din.v, din.g, din.beta))
    pool = din.pool.to(dev)
    idx = din.state_indices.to(dev)
    dout = torch.empty(args.decode_B, 1, din.v.shape[1], V, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    prefill = lambda: kda.chunk_prefill(q, k, v, g, beta, s0, None, out=o, final_state=sf, workspace=ws)
    decode = lambda: kda.decode(dq, dk, dv, dg, db, pool, idx, out=dout)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        prefill()
        if ev is not None:
            ev[1].record(stream)
        decode()
        if ev is not None:
            ev[2].record(stream)

    # Settle: the first calls after the host-side input generation run at
    # ramping clocks (the first 20 prefill calls measured up to 20% slower
    # than later ones), so the step runs untimed for a fixed 0.3 s of wall
    # clock before the W warmup steps.
    print("[bench] settle 0.3 s", file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.3:
        step()
        torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    pre = stats_us(pre_ms)
    dec = stats_us(dec_ms)
    pre_mean = pre["mean"] * 1e-3
    dec_mean = dec["mean"] * 1e-3

    pbytes = prefill_alg_bytes(B * T, H, HV, 1, True)
    pflops = prefill_alg_flops(B * T, HV)
    achieved_gbs = pbytes / (pre_mean * 1e-3) / 1e9
    mfma_tflops = pflops / (pre_mean * 1e-3) / 1e12
    t_hbm = pbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = pflops / (F16_PEAK_TFLOPS * 1e12)

    n_act = int((din.state_indices >= 0).sum())
    dbytes = decode_alg_bytes(n_act, args.decode_B - n_act, din.q.shape[1], din.v.shape[1])
    dec_gbs = dbytes / (dec_mean * 1e-3) / 1e9

    traffic = traffic_from_profiles()
    result = {
        "metric": METRIC,
        "value": B * T / (pre_mean * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"prefill B={B} H=HV={HV} T={T} K=V=128 (+ decode B={args.decode_B} H=HV=12 per step)",
            "global_batch": B,
            "seq_len": T,
            "parallelism": "single-gpu",
        },
        "roofline": {
            "kernel": "kda_chunk_prefill (intra_kernel<false, true> beside inter_kernel<32>, overlapped)",
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "timing": "HIP events on the launch stream around each call, back-to-back steps; the decode "
                  "follows a prefill whose >1 GB of traffic leaves it cache-cold",
        "prefill": {
            "event_us": pre,
            "alg_bytes": pbytes,
            "alg_flops": pflops,
            "mfma_tflops": mfma_tflops,
            "mfma_frac": mfma_tflops / F16_PEAK_TFLOPS,
            "attainable_frac": max(t_hbm, t_mfma) / (pre_mean * 1e-3),
        },
        "decode": {
            "B": args.decode_B,
            "active_rows": n_act,
            "event_us": dec,
            "alg_bytes": dbytes,
            "state_gbs": dec_gbs,
            "hbm_frac": dec_gbs / HBM_PEAK_GBS,
        },
    }
    if args.only_steps:
        if args.cpu_seconds > 0:
            result["cpu_baseline"] = cpu_baseline(pin, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return

    # Device kernel durations (no launch or inter-call gaps), and the same
    # calls after a 1 GiB cache-flushing write.
    print("[bench] device durations and cache-flushed timings", file=sys.stderr, flush=True)
    n_aux = max(5, args.steps // 2)
    # Device kernel durations (no launch or inter-call gaps) of the same
    # steps, from the committed rocprofv3 kernel trace when it was taken on
    # the current kernel sources.
    kt = kernel_trace_from_profiles()
    if kt:
        ku = kt["kernels_us"]
        for key, us, nbytes in (("prefill", kt.get("prefill_call_span_us"), pbytes),
                                ("decode", ku.get("decode_kernel"), dbytes)):
            kern = {n: v for n, v in ku.items() if (n.startswith("decode") == (key == "decode"))}
            result[key]["device_trace_us"] = {"us_per_call": us, "kernels": kern,
                                              "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS if us else None,
                                              "source": "profiles/kernel_trace_h96_t8192.json (" + kt["source"] +
                                                        ("; the prefill call's device span" if key == "prefill" else "") + ")"}
    else:
        result["prefill"]["device_trace_us"] = result["decode"]["device_trace_us"] = None
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.view(torch.float32).sum()
    pf = stats_us(time_events(torch, stream, prefill, n_aux, 1, flush))
    result["prefill"]["flushed_event_us"] = pf
    df = stats_us(time_events(torch, stream, decode, n_aux, 1, flush))
    result["decode"]["flushed_event_us"] = df
    result["decode"]["flushed_hbm_frac"] = dbytes / (df["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS
    result["cache_conditions"] = ("event_us: back-to-back steps (prefill then decode); flushed_event_us: "
                                  "a 1 GiB read (untimed) before every call, so each call starts with "
                                  "L2 and the 256 MB last-level cache holding none of its inputs")

    # The other workloads: each timed after a cache flush, with its
    # algorithmic bytes and the fraction of the HBM roofline.
    print("[bench] other workloads", file=sys.stderr, flush=True)
    configs = {}

    def prefill_line(inp, label, bound):
        a = [t.to(dev) if t is not None else None for t in (inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                              inp.initial_state, inp.cu_seqlens)]
        Bc, Tc, Hc, _ = inp.q.shape
        HVc = inp.v.shape[2]
        Nc = inp.cu_seqlens.numel() - 1 if inp.cu_seqlens is not None else Bc
        oc = torch.empty(Bc, Tc, HVc, V, dtype=torch.bfloat16, device=dev)
        sc = torch.empty(Nc, HVc, K, V, dtype=torch.float32, device=dev)
        wc = torch.empty(max(16, kda.workspace_size(Bc, Tc, Hc, HVc, Nc if inp.cu_seqlens is not None else 0)),
                         dtype=torch.uint8, device=dev)
        fn = lambda: kda.chunk_prefill(*a, out=oc, final_state=sc, workspace=wc)
        st = stats_us(time_events(torch, stream, fn, n_aux, 2, flush))
        nb = prefill_alg_bytes(Bc * Tc, Hc, HVc, Nc, inp.initial_state is not None)
        nf = prefill_alg_flops(Bc * Tc, HVc)
        part = kda.prefill_partition(Bc, HVc, Nc if inp.cu_seqlens is not None else 0)
        configs[label] = {"bound": bound, "partition": part, "flushed_event_us": st,
                          "tokens_per_s": Bc * Tc / (st["mean"] * 1e-6),
                          "alg_bytes": nb, "hbm_frac": nb / (st["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "mfma_frac": nf / (st["mean"] * 1e-6) / 1e12 / F16_PEAK_TFLOPS}

    prefill_line(synth.config0(), "prefill B=1 H=HV=1 T=128", "launch latency (0.26 MB)")
    prefill_line(synth.config1(), "prefill B=2 H=HV=8 T=1000 harsh decay", "latency / parallelism (26.7 MB)")
    c3 = synth.config3()
    prefill_line(c3, f"prefill varlen N=16 H=16 HV=32 T={c3.q.shape[1]}", "hbm")
    for Bd in (1, 8, 32, 256):
        di = synth.decode_config(Bd)
        da = [t.to(dev) for t in (di.q, di.k, di.v, di.g, di.beta)]
        dp = di.pool.to(dev)
        dx = di.state_indices.to(dev)
        do_ = torch.empty(Bd, 1, 12, V, dtype=torch.bfloat16, device=dev)
        st = stats_us(time_events(torch, stream, lambda: kda.decode(*da, dp, dx, out=do_), n_aux, 2, flush))
        na = int((di.state_indices >= 0).sum())
        nb = decode_alg_bytes(na, Bd - na, 12, 12)
        configs[f"decode B={Bd} H=HV=12"] = {
            "bound": "hbm" if Bd >= 256 else "launch latency",
            "active_rows": na, "flushed_event_us": st, "alg_bytes": nb,
            "hbm_frac": nb / (st["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del dp
    result["configs"] = configs
    del flush_buf

    # Prefill-to-decode handoff, timed on its own after the steps: the decode
    # workload's rows each hand a fresh fp32 state to their pool slot.  As
    # for the decode, a prefill runs before every launch, so each launch
    # meets the caches the way it would in serving and streams its states
    # from HBM.
    print("[bench] handoff", file=sys.stderr, flush=True)
    hstate, _, _ = synth.handoff_config(args.decode_B, slots=args.decode_B, HV=din.v.shape[1])
    hstate = hstate.to(dev)
    h_ms = time_events(torch, stream, lambda: kda.state_to_pool(hstate, pool, idx), args.steps, args.warmup,
                       prefill)
    h_mean = sum(h_ms) / len(h_ms)
    hbytes = handoff_alg_bytes(n_act, args.decode_B, din.v.shape[1])
    result["handoff"] = {
        "states": args.decode_B,
        "active": n_act,
        "event_us": stats_us(h_ms),
        "alg_bytes": hbytes,
        "gbs": hbytes / (h_mean * 1e-3) / 1e9,
        "hbm_frac": hbytes / (h_mean * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    # Packed decode (the page's serving-native inputs), timed the same way.
    print("[bench] packed decode", file=sys.stderr, flush=True)
    pk = synth.packed_decode_config(args.decode_B)
    pk_args = [t.to(dev) for t in (pk.mixed_qkv, pk.raw_gate, pk.raw_beta, pk.A_log, pk.dt_bias)]
    pk_pool = pk.pool.to(dev)
    pk_idx = pk.state_indices.to(dev)
    pk_out = torch.empty(args.decode_B, 1, pk.H, V, dtype=torch.bfloat16, device=dev)
    p_ms = time_events(torch, stream, lambda: kda.packed_decode(*pk_args, pk_pool, pk_idx, out=pk_out),
                       args.steps, args.warmup, prefill)
    p_mean = sum(p_ms) / len(p_ms)
    pk_act = int((pk.state_indices >= 0).sum())
    pkbytes = packed_decode_alg_bytes(pk_act, args.decode_B - pk_act, pk.H)
    result["packed_decode"] = {
        "B": args.decode_B,
        "active_rows": pk_act,
        "event_us": stats_us(p_ms),
        "alg_bytes": pkbytes,
        "gbs": pkbytes / (p_mean * 1e-3) / 1e9,
        "hbm_frac": pkbytes / (p_mean * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    del pk_pool
    # The two prefill partitions side by side: split (chunk-parallel kernel +
    # workspace + carry kernel) and fused (one workgroup per sequence and
    # value head, no workspace), on this workload (96 units), on the
    # 16-sequence varlen GQA batch (512 units) and on B=16 H=HV=64 T=2048
    # (1024 units); "auto" names the one kda_chunk_prefill runs.
    print("[bench] prefill partitions", file=sys.stderr, flush=True)

    def mean_us(fn, n):
        return stats_us(time_events(torch, stream, fn, n, args.warmup))["mean"]

    partitions = {}
    n_part = max(3, args.steps // 2)
    partitions[f"B=1 H=HV={HV} T={T}"] = {
        "units": B * HV,
        "auto": kda.prefill_partition(B, HV),
        "split_us": mean_us(lambda: kda.chunk_prefill_split(q, k, v, g, beta, s0, None, out=o, final_state=sf,
                                                            workspace=ws), n_part),
        # the same split form without room for the ready flags: the
        # sequential schedule (chunk kernel, then the two-workgroup carry)
        "split_sequential_us": mean_us(lambda: kda.chunk_prefill_split(
            q, k, v, g, beta, s0, None, out=o, final_state=sf,
            workspace=ws[:kda.workspace_size(B, T, H, HV) - flag_room(B, T, HV)]), n_part),
        "fused_us": mean_us(lambda: kda.chunk_prefill_fused(q, k, v, g, beta, s0, None, out=o, final_state=sf),
                            n_part),
    }
    c3a = [t.to(dev) for t in (c3.q, c3.k, c3.v, c3.g, c3.beta, c3.initial_state, c3.cu_seqlens)]
    T3, N3, H3, HV3 = c3.q.shape[1], c3.cu_seqlens.numel() - 1, c3.q.shape[2], c3.v.shape[2]
    o3 = torch.empty(1, T3, HV3, V, dtype=torch.bfloat16, device=dev)
    sf3 = torch.empty(N3, HV3, K, V, dtype=torch.float32, device=dev)
    ws3 = torch.empty(kda.workspace_size(1, T3, H3, HV3, N3), dtype=torch.uint8, device=dev)
    partitions[f"varlen N={N3} H={H3} HV={HV3} T={T3}"] = {
        "units": N3 * HV3,
        "auto": kda.prefill_partition(1, HV3, N3),
        "split_us": mean_us(lambda: kda.chunk_prefill_split(*c3a, out=o3, final_state=sf3, workspace=ws3), n_part),
        "fused_us": mean_us(lambda: kda.chunk_prefill_fused(*c3a, out=o3, final_state=sf3), n_part),
    }
    del c3a, o3, sf3, ws3
    c4 = synth.prefill_basic(5, 16, 2048, 64, 64, init="normal0.1", name="b16_h64_t2048")
    c4a = [t.to(dev) for t in (c4.q, c4.k, c4.v, c4.g, c4.beta, c4.initial_state)]
    o4 = torch.empty(16, 2048, 64, V, dtype=torch.bfloat16, device=dev)
    sf4 = torch.empty(16, 64, K, V, dtype=torch.float32, device=dev)
    ws4 = torch.empty(kda.workspace_size(16, 2048, 64, 64), dtype=torch.uint8, device=dev)
    partitions["B=16 H=HV=64 T=2048"] = {
        "units": 16 * 64,
        "auto": kda.prefill_partition(16, 64),
        "split_us": mean_us(lambda: kda.chunk_prefill_split(*c4a, None, out=o4, final_state=sf4, workspace=ws4),
                            n_part),
        "fused_us": mean_us(lambda: kda.chunk_prefill_fused(*c4a, None, out=o4, final_state=sf4), n_part),
    }
    del c4a, o4, sf4, ws4
    result["prefill_partitions"] = partitions
    result["backward"] = measure_backward(torch, synth, kda, pin, (q, k, v, g, beta, s0), stream,
                                          max(3, args.steps // 2), args.warmup)
    print("[bench] measured ceilings", file=sys.stderr, flush=True)
    del ws
    result["measured_ceilings"] = measured_ceilings(torch, dev)
    if args.cpu_seconds > 0:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pin, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
