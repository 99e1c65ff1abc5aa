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
  roofline     the prefill kernel against the HBM roofline (algorithmic
               bytes per launch / mean launch time, HIP events on the launch
               stream); traffic is filled from committed rocprofv3 counter
               summaries when they were taken on the current kernel source
  cpu_baseline the fp64 oracle (token-by-token form) on a bounded sample of
               the same prefill workload, on this host's cores
Only --gpus 1 is supported: the library runs on one GPU.
"""

import argparse
import hashlib
import json
import os
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


def decode_alg_bytes(B_act, B_inact, H, HV):
    """Active rows read and write their bf16 state slot and read q,k,v,g,beta
    and write o; inactive rows write zero o; plus the int32 indices."""
    per = 2 * K * V * 2 + 2 * K * 2 * H / HV + V * 2 + K * 4 + 2 + V * 2
    return B_act * HV * per + 4 * (B_act + B_inact) + B_inact * HV * V * 2


def source_hash(name):
    path = os.path.join(ROOT, "kda_gated_delta_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


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
    if rec.get("prefill_source_sha256_16") != source_hash("prefill.hip"):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, heads, seconds_hint):
    """Time the fp64 recurrent oracle on `heads` value heads of the prefill
    workload (all T tokens); scale to the full workload's tokens/s."""
    import numpy as np
    import oracle
    h = slice(0, heads)
    q = inp.q[:, :, h].float().numpy()
    k = inp.k[:, :, h].float().numpy()
    v = inp.v[:, :, h].float().numpy()
    g = inp.g[:, :, h].numpy()
    b = inp.beta[:, :, h].float().numpy()
    s0 = inp.initial_state[:, h].numpy()
    c0 = time.process_time()
    t0 = time.perf_counter()
    oracle.recurrent(q, k, v, g, b, s0)
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    T = inp.q.shape[1]
    HV = inp.v.shape[2]
    return {
        "value": T * heads / HV / wall,
        "unit": "tokens/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"fp64 token-by-token oracle on {heads} of {HV} value heads x all {T} tokens "
                  f"({wall:.1f} s); tokens/s scaled to all {HV} heads; host has {os.cpu_count()} cpus",
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
    args = ap.parse_args()
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
    if args.cpu_heads > 0:
        print(f"[bench] cpu oracle baseline on {args.cpu_heads} heads", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(pin, args.cpu_heads, 20)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
