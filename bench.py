"""Throughput of the S6 selective-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one selscan_fwd pass over one batch of the workload (default: one
Mamba-130M layer, batch 8, L 2048, D 1536, N 16, bf16 inputs, fp32 state,
SiLU(z) gate).  Inputs are seeded synthetic data, resident in HBM before the
timed region.  Several copies of the input set rotate between steps so that
consecutive steps do not find their inputs in the 256 MB last-level cache.

Prints one JSON line: elements (batch*L*dim) per second as ``value``, HBM GB/s
from the algorithmic bytes, the roofline entry of the scan kernel (average
launch time measured with HIP events on the launch stream), and the CPU
oracle timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def algorithmic_bytes(batch, L, dim, N, es, gate, with_last=False, with_h0=False):
    """Bytes the forward must move at least once: u, Delta (and z) read and y
    written per (b, l, d); B and C read per (b, l, n); A, D_skip and bias read
    once; h_last written (and h0 read) per (b, d, n) when used."""
    elems = batch * L * dim
    per_elem = (3 if gate else 2) * es + es
    b = elems * per_elem + 2 * batch * L * N * es + dim * N * 4 + 2 * dim * 4
    if with_last:
        b += batch * dim * N * 4
    if with_h0:
        b += batch * dim * N * 4
    return b


def cpu_baseline(w, inp_full, budget_s=15.0):
    """The oracle (untuned, OpenMP over (b, d)) on a bounded sample of the
    workload: whole batch rows, as many as fit in about ``budget_s``."""
    import oracle
    import selscan_inputs as si
    threads = oracle.default_threads()

    def rows(r0, r1):
        sl = slice(r0, r1)
        return si.FwdInputs(dtype=inp_full.dtype, batch=r1 - r0, L=inp_full.L, dim=inp_full.dim,
                            N=inp_full.N, u=si.Tensor(inp_full.u.value[sl]),
                            delta=si.Tensor(inp_full.delta.value[sl]),
                            Bm=si.Tensor(inp_full.Bm.value[sl]), Cm=si.Tensor(inp_full.Cm.value[sl]),
                            z=None if inp_full.z is None else si.Tensor(inp_full.z.value[sl]),
                            A=inp_full.A, D_skip=inp_full.D_skip, delta_bias=inp_full.delta_bias)

    t0 = time.perf_counter()
    oracle.fwd_inputs(rows(0, 1), threads=threads)
    t1 = time.perf_counter() - t0
    n_rows = int(max(1, min(w.batch - 1, budget_s / max(t1, 1e-3) - 1)))
    t0 = time.perf_counter()
    if n_rows >= 1 and w.batch > 1:
        oracle.fwd_inputs(rows(1, 1 + n_rows), threads=threads)
        dt = time.perf_counter() - t0
        done = n_rows
    else:
        dt, done = t1, 1
    elems = done * w.L * w.dim
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d batch rows of %s (%d elements, %.1f s wall, fp64, OpenMP)"
                      % (done, w.batch, w.name, elems, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba130m_layer")
    ap.add_argument("--rotate", type=int, default=4, help="input-set copies to rotate")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the scan shards over (batch, dim) "
              "with no exchange, so multi-GPU throughput is not measured here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import selscan_inputs as si
    import selective_state_space_selscan_amd as ss

    w = si.WORKLOADS[args.workload]
    if w.decode_steps:
        raise SystemExit("bench.py times the forward scan; pick a forward workload")
    dev = torch.device("cuda:0")
    inp = si.workload_fwd_inputs(w)
    base = si.fwd_tensors(inp, dev)
    sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                     for _ in range(args.rotate - 1)]
    es = 2 if w.dtype == si.BF16 else 4
    ys = [torch.empty((w.batch, w.L, w.dim), dtype=base["u"].dtype, device=dev)
          for _ in range(args.rotate)]
    hls = [torch.empty((w.batch, w.dim, w.N), dtype=torch.float32, device=dev)
           if w.want_last_state else None for _ in range(args.rotate)]
    code = ss.SELSCAN_BF16 if w.dtype == si.BF16 else ss.SELSCAN_F32
    ws_bytes = ss.selscan_fwd_workspace_bytes(w.batch, w.L, w.dim, w.N, code)
    wss = [torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
           for _ in range(args.rotate)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = sets[i % args.rotate]
        ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, None, return_last_state=w.want_last_state,
                       y=ys[i % args.rotate], h_last=hls[i % args.rotate],
                       workspace=wss[i % args.rotate], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    elems = w.batch * w.L * w.dim
    ms_per_step = 1e3 * wall / args.steps
    kernel_ms = float(np.mean(launch_ms))
    abytes = algorithmic_bytes(w.batch, w.L, w.dim, w.N, es, w.gate, w.want_last_state)
    achieved = abytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": "selective-scan fwd elements(B*L*D)/s and HBM GB/s (% of MI355X peak), 1 GPU",
        "value": elems / (ms_per_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == si.BF16 else "f32",
        "data": "synthetic (seeded; u,B,C,z ~ N(0,1), Delta_raw ~ N(0,0.5^2), "
                "dt log-uniform [1e-3,0.1], A=-(n+1), D=1)",
        "config": {"workload": w.name, "batch": w.batch, "L": w.L, "dim": w.dim, "N": w.N,
                   "gate": w.gate, "state": "fp32", "rotating_input_sets": args.rotate},
        "hbm_gbps": abytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": abytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "kernel_ms": {"mean": kernel_ms, "p10": float(np.percentile(launch_ms, 10)),
                      "p50": float(np.median(launch_ms)),
                      "p90": float(np.percentile(launch_ms, 90))},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": abytes},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
