"""Benchmark of the KDA forward hot path on one MI355X.

One step = one chunked prefill of the at-scale workload (B=1, H=HV=96,
T=8192, K=V=128, zero fp32 initial state) followed by one decode step of the
B=256 decode workload (H=HV=12, bf16 state pool [1024,12,128,128], 1/8 of the
rows inactive).  Inputs are synthetic (seeded, generated on the host, copied
to HBM before timing).  The prefill's 1.2 GB of traffic evicts the decode
pool's slots from the 256 MB last-level cache between decode calls, so the
decode runs cache-cold.

Prints one JSON line:
  value        prefill tokens/s (T / mean prefill kernel time)
  roofline     the prefill entry point -- its two kernels, intra_kernel then
               inter_kernel, timed together by HIP events on the launch
               stream -- against the HBM roofline: algorithmic bytes per
               call / mean call time.  traffic is the measured HBM bytes per
               call from the committed rocprofv3 counter summary when that
               was taken on the current kernel source, else null
  handoff,     the prefill-to-decode handoff (256 x 12 fp32 states into the
  packed_decode  pool) and the packed-input decode (B=256, H=12), each timed
               after the steps with a prefill before every launch, so they
               too meet the caches the way they would in serving
  prefill_partitions  mean call time of the split and the fused prefill
               partitions on this workload, on the 16-sequence varlen GQA
               batch (512 units) and on B=16 H=HV=64 T=2048 (1024 units)
  cpu_baseline the fp64 oracle (token-by-token form) on a bounded sample of
               the same prefill workload, on this host's cores
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
    state and final-state gradient fp32) and float32 gradients written once
    (dq, dk, dv, dg, dbeta, d_initial_state)."""
    per_tok = H * 2 * K * 2 + HV * (V * 2 + K * 4 + 2 + V * 2)          # inputs
    per_tok += H * 2 * K * 4 + HV * (V * 4 + K * 4 + 4)                 # gradients
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


def cpu_baseline(inp, heads, target_s):
    """Time the fp64 recurrent oracle on a bounded sample of the prefill
    workload: the first value heads over the first tokens, sized from pilot
    runs so that the timed run takes about `target_s` seconds.  Reported as
    tokens/s of the full workload (all value heads)."""
    import numpy as np
    import oracle
    h = slice(0, heads)
    T = inp.q.shape[1]
    HV = inp.v.shape[2]

    def run(n):
        q = inp.q[:, :n, h].float().numpy()
        k = inp.k[:, :n, h].float().numpy()
        v = inp.v[:, :n, h].float().numpy()
        g = inp.g[:, :n, h].numpy()
        b = inp.beta[:, :n, h].float().numpy()
        s0 = inp.initial_state[:, h].numpy()
        c0 = time.process_time()
        t0 = time.perf_counter()
        oracle.recurrent(q, k, v, g, b, s0)
        return time.perf_counter() - t0, time.process_time() - c0

    # Pilot on `heads` heads over all tokens (the oracle is fast enough on the
    # hosts here), then widen the head count so the timed run lands near
    # target_s; on a slow host shorten the token range instead.
    n = min(T, 256)
    w, _ = run(n)
    n = int(min(T, max(n, n * target_s / max(w, 1e-6))))
    if n == T:
        w, _ = run(n)
        heads = int(min(HV, max(heads, heads * target_s / max(w, 1e-6))))
        h = slice(0, heads)
    wall, cpu = run(n)
    return {
        "value": n * heads / HV / wall,
        "unit": "tokens/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 token-by-token oracle on the prefill workload's first {heads} of {HV} value heads "
                  f"x first {n} of {T} tokens ({wall:.1f} s wall, {cpu:.1f} s cpu); tokens/s scaled to all "
                  f"{HV} heads; host reports {os.cpu_count()} cpus",
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

    def pick(d, key):
        vals = [v for k, v in d.items() if key in k]
        if not vals:
            raise SystemExit(f"no {key} dispatches in the counter file")
        return vals[0]

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
    total = 0.0
    for key in ("intra_kernel", "inter_kernel"):
        fb = pick(f, key) / f_scale * 1024.0
        wb = pick(w, key) / w_scale * 1024.0
        rec["kernels"][key] = {"fetch_bytes": fb, "write_bytes": wb}
        total += fb + wb
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--T", type=int, default=8192)
    ap.add_argument("--H", type=int, default=96)
    ap.add_argument("--decode-B", type=int, default=256)
    ap.add_argument("--cpu-heads", type=int, default=8, help="value heads in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target wall time of the CPU-oracle sample")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the backward of the prefill workload (for profiling)")
    ap.add_argument("--only-steps", action="store_true",
                    help="time only the steps (prefill + decode); skip the handoff, packed decode and "
                         "partition measurements (for profiler runs that average per kernel name)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=6, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                           "COPY_WRITE_CSV", "COPY_BYTES", "OUT_JSON"),
                    help="only summarise rocprofv3 counter files into the traffic record")
    args = ap.parse_args()
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
    if args.only_backward:
        torch.cuda.synchronize()
        bw = measure_backward(torch, synth, kda, pin, (q, k, v, g, beta, s0), torch.cuda.current_stream(),
                              args.steps, args.warmup)
        print(json.dumps({"backward": bw}), flush=True)
        return

    din = synth.decode_config(args.decode_B)
    dq, dk, dv, dg, db = (t.to(dev) for t in (din.q, din.k, din.v, din.g, din.beta))
    pool = din.pool.to(dev)
    idx = din.state_indices.to(dev)
    dout = torch.empty(args.decode_B, 1, din.v.shape[1], V, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda.chunk_prefill(q, k, v, g, beta, s0, None, out=o, final_state=sf, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        kda.decode(dq, dk, dv, dg, db, pool, idx, out=dout)
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
    pre_mean = sum(pre_ms) / len(pre_ms)
    dec_mean = sum(dec_ms) / len(dec_ms)
    pre_sorted = sorted(pre_ms)

    n_seq = 1
    pbytes = prefill_alg_bytes(B * T, H, HV, n_seq, True)
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
            "kernel": "kda_chunk_prefill (intra_kernel + inter_kernel)",
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "prefill": {
            "kernel_us_mean": pre_mean * 1e3,
            "kernel_us_p10": pre_sorted[len(pre_sorted) // 10] * 1e3,
            "kernel_us_p90": pre_sorted[(9 * len(pre_sorted)) // 10] * 1e3,
            "alg_bytes": pbytes,
            "alg_flops": pflops,
            "mfma_tflops": mfma_tflops,
            "mfma_frac": mfma_tflops / F16_PEAK_TFLOPS,
            "attainable_frac": max(t_hbm, t_mfma) / (pre_mean * 1e-3),
        },
        "decode": {
            "B": args.decode_B,
            "active_rows": n_act,
            "kernel_us_mean": dec_mean * 1e3,
            "alg_bytes": dbytes,
            "state_gbs": dec_gbs,
            "hbm_frac": dec_gbs / HBM_PEAK_GBS,
        },
    }
    if args.only_steps:
        result["cpu_baseline"] = cpu_baseline(pin, args.cpu_heads, args.cpu_seconds) if args.cpu_heads > 0 else None
        print(json.dumps(result), flush=True)
        return

    # Prefill-to-decode handoff, timed on its own after the steps: the decode
    # workload's rows each hand a fresh fp32 state to their pool slot.  As
    # for the decode, a prefill runs before every launch, so each launch
    # meets the caches the way it would in serving and streams its states
    # from HBM.
    print("[bench] handoff", file=sys.stderr, flush=True)
    hstate, _, _ = synth.handoff_config(args.decode_B, slots=args.decode_B, HV=din.v.shape[1])
    hstate = hstate.to(dev)
    h_ev = []
    for i in range(args.warmup + args.steps):
        kda.chunk_prefill(q, k, v, g, beta, s0, None, out=o, final_state=sf, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.state_to_pool(hstate, pool, idx)
        e1.record(stream)
        if i >= args.warmup:
            h_ev.append((e0, e1))
    torch.cuda.synchronize()
    h_ms = [a.elapsed_time(b) for a, b in h_ev]
    h_mean = sum(h_ms) / len(h_ms)
    hbytes = handoff_alg_bytes(n_act, args.decode_B, din.v.shape[1])
    result["handoff"] = {
        "states": args.decode_B,
        "active": n_act,
        "kernel_us_mean": h_mean * 1e3,
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
    p_ev = []
    for i in range(args.warmup + args.steps):
        kda.chunk_prefill(q, k, v, g, beta, s0, None, out=o, final_state=sf, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.packed_decode(*pk_args, pk_pool, pk_idx, out=pk_out)
        e1.record(stream)
        if i >= args.warmup:
            p_ev.append((e0, e1))
    torch.cuda.synchronize()
    p_mean = sum(a.elapsed_time(b) for a, b in p_ev) / len(p_ev)
    pk_act = int((pk.state_indices >= 0).sum())
    pkbytes = packed_decode_alg_bytes(pk_act, args.decode_B - pk_act, pk.H)
    result["packed_decode"] = {
        "B": args.decode_B,
        "active_rows": pk_act,
        "kernel_us_mean": p_mean * 1e3,
        "alg_bytes": pkbytes,
        "gbs": pkbytes / (p_mean * 1e-3) / 1e9,
        "hbm_frac": pkbytes / (p_mean * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    del pk_pool
    # The two prefill partitions side by side: split (the entry point timed
    # above: chunk-parallel kernel + workspace + carry kernel) and fused (one
    # workgroup per sequence and value head, no workspace), on this workload
    # (96 units) and on the 16-sequence varlen GQA batch (512 units).
    print("[bench] prefill partitions", file=sys.stderr, flush=True)

    def time_calls(fn, n):
        evs = []
        for i in range(args.warmup + n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            if i >= args.warmup:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3

    partitions = {}
    n_part = max(3, args.steps // 2)
    partitions[f"B=1 H=HV={HV} T={T}"] = {
        "units": B * HV,
        "split_us": time_calls(lambda: kda.chunk_prefill(q, k, v, g, beta, s0, None, out=o, final_state=sf,
                                                         workspace=ws), n_part),
        "fused_us": time_calls(lambda: kda.chunk_prefill_fused(q, k, v, g, beta, s0, None, out=o,
                                                               final_state=sf), n_part),
    }
    c3 = synth.config3()
    c3a = [t.to(dev) for t in (c3.q, c3.k, c3.v, c3.g, c3.beta, c3.initial_state, c3.cu_seqlens)]
    T3, N3, H3, HV3 = c3.q.shape[1], c3.cu_seqlens.numel() - 1, c3.q.shape[2], c3.v.shape[2]
    o3 = torch.empty(1, T3, HV3, V, dtype=torch.bfloat16, device=dev)
    sf3 = torch.empty(N3, HV3, K, V, dtype=torch.float32, device=dev)
    ws3 = torch.empty(kda.workspace_size(1, T3, H3, HV3, N3), dtype=torch.uint8, device=dev)
    partitions[f"varlen N={N3} H={H3} HV={HV3} T={T3}"] = {
        "units": N3 * HV3,
        "split_us": time_calls(lambda: kda.chunk_prefill(*c3a, out=o3, final_state=sf3, workspace=ws3), n_part),
        "fused_us": time_calls(lambda: kda.chunk_prefill_fused(*c3a, out=o3, final_state=sf3), n_part),
    }
    del c3a, o3, sf3, ws3
    # Many equal sequences: B=16, H=HV=64, T=2048 (1024 units).
    c4 = synth.prefill_basic(5, 16, 2048, 64, 64, init="normal0.1", name="b16_h64_t2048")
    c4a = [t.to(dev) for t in (c4.q, c4.k, c4.v, c4.g, c4.beta, c4.initial_state)]
    o4 = torch.empty(16, 2048, 64, V, dtype=torch.bfloat16, device=dev)
    sf4 = torch.empty(16, 64, K, V, dtype=torch.float32, device=dev)
    ws4 = torch.empty(kda.workspace_size(16, 2048, 64, 64), dtype=torch.uint8, device=dev)
    partitions["B=16 H=HV=64 T=2048"] = {
        "units": 16 * 64,
        "split_us": time_calls(lambda: kda.chunk_prefill(*c4a, None, out=o4, final_state=sf4, workspace=ws4), n_part),
        "fused_us": time_calls(lambda: kda.chunk_prefill_fused(*c4a, None, out=o4, final_state=sf4), n_part),
    }
    del c4a, o4, sf4, ws4
    result["prefill_partitions"] = partitions
    result["backward"] = measure_backward(torch, synth, kda, pin, (q, k, v, g, beta, s0), stream,
                                          max(3, args.steps // 2), args.warmup)
    if args.cpu_heads > 0:
        print(f"[bench] cpu oracle baseline on {args.cpu_heads} heads", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pin, args.cpu_heads, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
