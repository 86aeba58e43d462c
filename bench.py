"""Throughput of the S6 selective-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --pmc-run            # workload for rocprofv3 --pmc (see below)
    python bench.py --pmc-run --pass bwd # the same for the backward
    python bench.py --parse-pmc FETCH_DIR WRITE_DIR   # -> profiles/traffic_<workload>.json
    python bench.py --pass bwd           # the backward (selscan_bwd) on the same workload
    python bench.py --variant zoh,rev,conv4   # forward variants through selscan_fwd_ex
    python bench.py --pass bwd --variant zoh,rev,conv4   # their backward (selscan_bwd_ex)
    python bench.py --pass fwdbwd        # forward + backward reusing its part state
    python bench.py --pass fwdbwd --keep-checkpoints   # ... and its checkpoints

One step = one selscan_fwd call over one batch of the workload.  The default
workload is one Mamba-130M layer: batch 8, L 2048, D 1536, N 16, bf16 inputs,
fp32 state, SiLU(z) gate.  Inputs are seeded synthetic data, resident in HBM
before the timed region.  Several copies of the input set rotate between
steps so that consecutive steps do not find their inputs in the 256 MB
last-level cache.

The JSON line carries:
  value      elements (batch*L*dim) per second over the timed steps;
  roofline   the forward call (summary, carry and main passes) against the VALU
             roofline: the path is bound by fp32 vector arithmetic, not by HBM
             (see algorithmic_valu_slots).  The call's average duration is
             the interval between two HIP events recorded on the launch
             stream around the timed steps, divided by their number;
  call_ms    that average, and the spread of single calls timed afterwards
             (50 more calls, each between its own pair of events);
  traffic    HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
             scaled by the same counters on a plain 1 GiB copy, read from
             profiles/traffic_<workload>.json if the kernel sources are
             unchanged since it was taken, else null;
  hbm_*      algorithmic bytes per call / step time, against the 8 TB/s peak;
  device_copy_gbps  a plain 512 MiB device copy timed in the same run, for
             context (what HBM delivers to a copy on this machine);
  cpu_baseline  the CPU oracle (fp64, OpenMP) on a bounded sample.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# fp32 vector issue rate without packed instructions: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz = 39.3e12 lane-operations per second (one FMA = one slot).
VALU_PEAK_SLOTS = 256 * 4 * 16 * 2.4e9
COPY_CAL_BYTES = 1 << 30


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


def algorithmic_valu_slots(N, gate, es, general_a=False, flags=0, conv_k=0):
    """fp32 VALU issue slots one (b, l, d) element needs on gfx950 without
    packed instructions.  A transcendental (exp2, log2, rcp) takes two slots.
    For A of the S4D-real form (A[d,n] = (n+1) A[d,0], every workload here):
      per state n: A_bar by one multiply (power chain), Delta*u*B (1), state
                   FMA (1), readout FMA (1)                        -> 4 N
      per element: widen u, Delta (2 if bf16), bias add (1), softplus (exp,
                   log: 4 slots, + 2), Delta*u (1), r = exp(Delta A0) (3),
                   D*u (1), round y (1 if bf16)
      gate:        widen z (1 if bf16), SiLU (exp, rcp: 4 slots, + 2), y*g (1)
    For a general A (general_a), A_bar = exp2(Delta A[d,n] log2 e) per state:
    a multiply and an exp2 (3 slots) in place of the power chain's multiply,
    and no r: 6 N + the per-element work less 3.
    Variants (``flags``, ``conv_k`` as for selscan_fwd_ex; the power chain):
      reverse:   addressing only                                    -> + 0
      exact ZOH: B_bar_n = c_n B_n with c_n = em S_n / (n+1), S_n the running
                 sum of the powers: per state the sum, S_n B_n and the scale
                 (3); per element em = (r - 1) / A[d,0] with its series
                 branch (9) in place of Delta*u (1)                -> + 3 N + 8
      conv:      k taps of the causal conv (k FMAs) and SiLU (exp, rcp: 4
                 slots, + 2) of the scan input                     -> + k + 6"""
    bf = 1 if es == 2 else 0
    per = 4 * N + 2 * bf + 1 + 6 + 1 + 3 + 1 + bf
    if gate:
        per += bf + 6 + 1
    if general_a:
        assert not flags & VARIANT_FLAGS["zoh"], "general A with exact ZOH is not counted"
        per += 2 * N - 3
    if flags & VARIANT_FLAGS["zoh"]:
        per += 3 * N + 8
    if conv_k:
        per += conv_k + 6
    return per


# The sources of the forward kernels the counters are taken on.
FWD_KERNEL_SOURCES = ("fwd_stream.hip", "fwd_stream_impl.hpp", "buffer_io.hpp", "device_math.hpp")


def source_digest():
    h = hashlib.sha256()
    for name in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "selective_state_space_selscan_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def load_traffic(workload):
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("bytes_per_call")


def cpu_model():
    """The host CPU's model name (as lscpu reports it), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp_full, cpu_budget_s=15.0):
    """The oracle (untuned, OpenMP over (b, d)) on the workload, repeated whole
    until about ``cpu_budget_s`` seconds of CPU time (all threads) are spent."""
    import oracle
    threads = oracle.default_threads()
    elems_per_pass = w.batch * w.L * w.dim
    c0, t0 = time.process_time(), time.perf_counter()
    passes = 0
    while True:
        oracle.fwd_inputs(inp_full, threads=threads)
        passes += 1
        if time.process_time() - c0 >= cpu_budget_s or passes >= 1000:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    return {"value": passes * elems_per_pass / wall, "unit": "elements/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d full pass(es) of %s (%d elements each), %.1f s wall, %.1f s CPU, "
                      "fp64 sequential recurrence, OpenMP over (b, d)"
                      % (passes, w.name, elems_per_pass, wall, cpu)}


def make_inputs(w, dev, rotate):
    import torch

    import selscan_inputs as si
    inp = si.workload_fwd_inputs(w)
    base = si.fwd_tensors(inp, dev)
    sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                     for _ in range(rotate - 1)]
    return inp, sets


def pmc_run(w, which="fwd", reps=3, warmup=200):
    """Workload for the counter runs: one plain 1 GiB device copy (the
    calibration), ``warmup`` calls (the clocks ramp up), then ``reps`` calls,
    the ones the counters are read on: forward calls, or with ``which`` =
    "bwd" backward calls as ``--pass bwd`` times them (dy seeded, no
    dh_last, one workspace)."""
    import torch

    import selscan_inputs as si
    import selective_state_space_selscan_amd as ss
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    _, sets = make_inputs(w, dev, 1)
    t = sets[0]
    if which == "bwd":
        rng = np.random.default_rng([w.seed, 4242])
        dy = torch.from_numpy(rng.standard_normal((w.batch, w.L, w.dim), dtype=np.float32))
        dy = dy.to(dev).to(t["u"].dtype)
        code = ss.SELSCAN_BF16 if w.dtype == si.BF16 else ss.SELSCAN_F32
        ws = torch.empty(ss.selscan_bwd_workspace_bytes(w.batch, w.L, w.dim, w.N, code),
                         dtype=torch.uint8, device=dev)
        for _ in range(warmup + reps):
            ss.selscan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"], t["z"],
                           t["delta_bias"], True, None, None, workspace=ws)
    else:
        for _ in range(warmup + reps):
            ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                           t["delta_bias"], True, None, return_last_state=w.want_last_state)
    torch.cuda.synchronize()
    print("pmc-run done", w.name, which, warmup, reps, flush=True)


def parse_pmc(w, fetch_dir, write_dir, reps=3):
    """Per-call HBM bytes from the two counter runs of ``pmc_run``."""
    import csv

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        vals = {}
        for fpath in files:
            for r in csv.DictReader(open(fpath)):
                if r["Counter_Name"] == counter:
                    key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return sorted(vals.items())

    out = {}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = per_kernel(d, counter)
        # the calibration copy is the largest copyBuffer dispatch (1 GiB)
        copy = sorted((v for (i, k), v in rows if "copyBuffer" in k), reverse=True)
        scan = [(k, v) for (i, k), v in rows if "selscan" in k]
        # the last reps calls (after the warmup calls): reps x the kernels of a call
        scan = scan[-reps * len({k for k, _ in scan}):]
        factor = COPY_CAL_BYTES / (copy[0] * 1024.0) if copy and copy[0] > 0 else None
        kib_per_call = sum(v for _, v in scan) / reps
        out[name] = {"counter": counter, "kib_per_call_raw": kib_per_call,
                     "copy_kib_raw": copy[0] if copy else None, "copy_factor": factor,
                     "bytes_per_call": None if factor is None else kib_per_call * 1024.0 * factor,
                     "kernels": sorted({k.replace("(anonymous namespace)::", "").split("(")[0]
                                        for k, _ in scan})}
    total = (out["fetch"]["bytes_per_call"] or 0) + (out["write"]["bytes_per_call"] or 0)
    res = {"workload": w.name, "source_sha256": source_digest(), "bytes_per_call": total,
           "fetch": out["fetch"], "write": out["write"],
           "algorithmic_bytes_per_call": algorithmic_bytes(
               w.batch, w.L, w.dim, w.N, 2 if w.dtype == "bf16" else 4, w.gate,
               w.want_last_state)}
    with open(traffic_file(w.name), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def decode_bytes(batch, dim, N, es, gate):
    """Bytes one decode step must move: the fp32 state read and written once
    (8 B per (b, d, n)), u, Delta (and z) read and y written per (b, d), B and C
    per (b, n), A, D and bias once."""
    return (batch * dim * N * 8 + batch * dim * ((3 if gate else 2) * es + es)
            + 2 * batch * N * es + dim * N * 4 + 2 * dim * 4)


def bench_decode(w, steps, warmup, ramp_ms=0.0):
    """Decode: ``steps`` single-token selscan_state_update calls on the resident
    fp32 state (batch, dim, N).  Warm: back-to-back steps, the 84 MB state may
    stay in the 256 MB last-level cache.  Cold: a 1 GiB buffer is read before
    each timed step, so the state comes from HBM.  (Writing the buffer instead
    would leave the cache full of dirty lines whose write-back then lands in
    the timed step.)"""
    import torch

    import selscan_inputs as si
    import selective_state_space_selscan_amd as ss
    dev = torch.device("cuda:0")
    A, D, bias = (torch.from_numpy(x).to(dev) for x in si.decode_params(w))
    ins = [si.step_tensors(st, w.dtype, dev) for st in si.decode_block(w, 0, 8)]
    state = torch.zeros((w.batch, w.dim, w.N), dtype=torch.float32, device=dev)
    ys = [torch.empty((w.batch, w.dim), dtype=ins[0]["u"].dtype, device=dev) for _ in ins]
    stream = torch.cuda.current_stream(dev)
    es = 2 if w.dtype == si.BF16 else 4

    def step(i):
        t = ins[i % len(ins)]
        ss.selscan_state_update(state, t["u"], t["delta"], A, t["Bm"], t["Cm"], D, t["z"], bias,
                                True, y=ys[i % len(ins)], stream=stream)

    ramp = clock_ramp(step, ramp_ms)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    flush.fill_(1.0)
    for i in range(min(steps, 50)):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold_ms = float(np.mean(cold))
    nb = decode_bytes(w.batch, w.dim, w.N, es, w.gate)
    elems = w.batch * w.dim
    res = {
        "metric": "selective-scan decode step (selscan_state_update) elements(batch*dim)/s, 1 GPU",
        "value": elems * steps / wall, "unit": "elements/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": 1e3 * wall / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == si.BF16 else "f32",
        "data": "synthetic (seeded per step)",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "N": w.N,
                   "state": "fp32 resident"},
        "clock_ramp": {"calls": ramp[0], "ms": ramp[1]},
        "step_ms_warm": warm_ms, "step_ms_cold": cold_ms,
        "device_copy_gbps": device_copy_gbps(dev),
        "roofline": {"bound": "hbm", "achieved": nb / (cold_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": nb / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "state_update_kernel, cold last-level cache",
                     "algorithmic_bytes_per_step": nb,
                     "warm_gbps": nb / (warm_ms * 1e-3) / 1e9},
    }
    print(json.dumps(res), flush=True)


def clock_ramp(step, ramp_ms):
    """Untimed steps for at least ``ramp_ms`` of wall time before the warmup
    steps.  An idle GPU runs its first milliseconds of work at lower clocks
    (the 130M-layer forward with 5 warmup calls: 139 us per call over the
    next 20, rising from 134 to 145; after 250 ms of calls 122 us, falling
    to 119), so a short warmup alone would time the ramp rather than the
    kernels.  Returns (calls, ms)."""
    import torch

    if ramp_ms <= 0:
        return 0, 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    calls = 0
    while (time.perf_counter() - t0) * 1e3 < ramp_ms:
        for _ in range(64):
            step(calls)
            calls += 1
        torch.cuda.synchronize()
    return calls, (time.perf_counter() - t0) * 1e3


def timed_steps(step, steps, warmup, stream, percall=50, ramp_ms=0.0):
    """A clock ramp of ``ramp_ms`` (clock_ramp), ``warmup`` untimed steps,
    then exactly ``steps`` steps back to back,
    bracketed by a synchronize on both sides (host clock) and by HIP events on
    the launch stream (device clock): the average call duration is the
    interval from the first event to the last / ``steps``.  Events also mark
    the quarters of the timed steps (when there are at least 4), so the mean
    call of each quarter shows whether the clocks were still ramping.  Then
    ``percall`` further steps, each between its own pair of events, for the
    spread of single calls; they are not part of the timed region (an event
    pair per call adds a small bubble of its own).  Returns (wall s, mean
    call ms, per-call ms array, mean call ms per quarter, (ramp calls, ramp
    ms))."""
    import torch

    ramp = clock_ramp(step, ramp_ms)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    marks = sorted({0, steps} | ({steps * q // 4 for q in range(1, 4)} if steps >= 4 else set()))
    ev = {m: torch.cuda.Event(enable_timing=True) for m in marks}
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step(warmup + i)
        if i + 1 in ev:
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_mean = ev[0].elapsed_time(ev[steps]) / steps
    quarters = [ev[m0].elapsed_time(ev[m1]) / (m1 - m0) for m0, m1 in zip(marks, marks[1:])]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(percall)]
    for i, (x, y) in enumerate(ev):
        x.record(stream)
        step(warmup + steps + i)
        y.record(stream)
    torch.cuda.synchronize()
    return wall, call_mean, np.array([x.elapsed_time(y) for x, y in ev]), quarters, ramp


def device_copy_gbps(dev, nbytes=1 << 29, reps=10):
    """Same-run context for the HBM figures: a device-to-device copy of
    ``nbytes`` (read + write counted), median over ``reps`` copies timed with
    HIP events, after the workload's own timing."""
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = []
    while len(ms) < reps:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    return 2 * nbytes / (float(np.median(ms)) * 1e-3) / 1e9


def bwd_valu_slots(N, gate, es, flags=0, conv_k=0, general_a=False):
    """fp32 VALU slots per (b, l, d) element of the backward as built, counted
    from the inner loops of its main pass (the summary and checkpoint passes
    and the carries are extra work of the recomputation scheme, not counted;
    a transcendental counts two slots).  Per state n:
      Euler B_bar (plain, reverse):   recompute 3 (A_bar by the power chain,
        Delta u B, state FMA); adjoint step 11 (lambda, readout, A_bar h_{t-1},
        its product with lambda, the dDelta and dA sums, lambda.B, the dB and
        dC terms, A_bar, the carry); the sums of dB and dC over the
        wave's lanes 2 (their adds; the lane exchanges come on top) -> 16 N
      general A (Euler): A_bar = exp2(Delta A[d,n] log2 e) per state in the
        recompute and in the adjoint step (a multiply and an exp2, 3 slots,
        in place of the power chain's multiply)                   -> 20 N
      exact ZOH: recompute 14 (the coefficient (e - 1)/A with its series
        branch: 9, times u B: 2); adjoint 40 (the coefficient again, its
        derivative in A with its series branch: 13, and the extra terms of
        dDelta and dA); the lane sums 2                           -> 56 N
    Per element about 60 (softplus and sigmoid twice, SiLU and its derivative,
    widening, the per-element gradients and stores); the conv prologue adds
    48: the conv and SiLU of the scan input in the summary and checkpoint
    passes (10 each; the main pass reads the checkpoint pass's fp32 output),
    and the epilogue's conv backward (28: the pre-activation again, its
    sigmoid, SiLU', the dconv_w and dconv_b sums and the transposed conv of
    dx)."""
    if general_a:
        assert not flags & VARIANT_FLAGS["zoh"], "general A with exact ZOH is not counted"
    per_n = 56 if flags & VARIANT_FLAGS["zoh"] else (20 if general_a else 16)
    return per_n * N + 60 + (48 if conv_k else 0)


def bench_bwd(w, args):
    """``steps`` selscan_bwd calls on the workload (upstream gradient dy
    seeded, no dh_last), inputs resident in HBM, one workspace.  With
    ``--pass fwdbwd`` a step is a training step's pair instead: selscan_fwd
    into the workspace, then selscan_bwd_ex reading the forward's part state
    from it (SELSCAN_FLAG_REUSE_FWD_STATE; plain or reverse alone)."""
    import torch

    import selscan_inputs as si
    import selective_state_space_selscan_amd as ss
    dev = torch.device("cuda:0")
    inp, sets = make_inputs(w, dev, 1)
    t = sets[0]
    general_a = args.a_form == "general"
    if general_a:
        t["A"] = torch.from_numpy(si.perturbed_A(w.dim, w.N, w.seed)).to(dev)
    rng = np.random.default_rng([w.seed, 4242])
    dy = torch.from_numpy(rng.standard_normal((w.batch, w.L, w.dim), dtype=np.float32)).to(dev)
    dy = dy.to(t["u"].dtype)
    code = ss.SELSCAN_BF16 if w.dtype == si.BF16 else ss.SELSCAN_F32
    ws = torch.empty(ss.selscan_bwd_workspace_bytes(w.batch, w.L, w.dim, w.N, code),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    vflags, vconv = parse_variant(args.variant)
    conv_w = conv_b = None
    if vconv:
        cw, cb = si.conv_params(w.dim, vconv, w.seed)
        conv_w, conv_b = torch.from_numpy(cw).to(dev), torch.from_numpy(cb).to(dev)
    pair = args.which == "fwdbwd"
    if pair and (vconv or vflags & ~ss.SELSCAN_FLAG_REVERSE):
        raise SystemExit("bench.py: --pass fwdbwd runs the plain path or 'rev' alone")
    keep = bool(getattr(args, "keep_checkpoints", False))
    if keep and (not pair or vflags & ~ss.SELSCAN_FLAG_REVERSE):
        raise SystemExit("bench.py: --keep-checkpoints goes with --pass fwdbwd, plain or 'rev'")
    kflag = ss.SELSCAN_FLAG_KEEP_CHECKPOINTS if keep else 0
    y = torch.empty_like(t["u"])

    def step(i):
        if pair:
            ss.selscan_fwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                              t["delta_bias"], True, None, flags=vflags | kflag, y=y,
                              workspace=ws, stream=stream)
            ss.selscan_bwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"],
                              t["z"], t["delta_bias"], True, None, None,
                              flags=vflags | ss.SELSCAN_FLAG_REUSE_FWD_STATE | kflag,
                              workspace=ws, stream=stream)
            return
        if args.variant:
            ss.selscan_bwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"],
                              t["z"], t["delta_bias"], True, None, None, flags=vflags,
                              conv_weight=conv_w, conv_bias=conv_b, workspace=ws, stream=stream)
            return
        ss.selscan_bwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], dy, t["D_skip"], t["z"],
                       t["delta_bias"], True, None, None, workspace=ws, stream=stream)

    wall, call_mean, call_ms, quarters, ramp = timed_steps(step, args.steps, args.warmup, stream,
                                                             ramp_ms=args.ramp_ms)
    es = 2 if w.dtype == si.BF16 else 4
    elems = w.batch * w.L * w.dim
    slots_el = bwd_valu_slots(w.N, w.gate, es, vflags, vconv, general_a) + (
        algorithmic_valu_slots(w.N, w.gate, es, general_a) if pair else 0)
    slots = slots_el * elems
    # bytes the backward must move: the forward's inputs once, dy, and the
    # gradients du, ddelta, dz (dtype) and dB, dC (fp32) once
    nb = (elems * ((3 if w.gate else 2) * es + es + (3 if w.gate else 2) * es)
          + 2 * w.batch * w.L * w.N * (es + 4) + w.dim * w.N * 8 + 4 * w.dim * 4)
    if pair:
        nb += algorithmic_bytes(w.batch, w.L, w.dim, w.N, es, w.gate)
    achieved = slots / (call_mean * 1e-3) / 1e9
    res = {
        "metric": "selective-scan %s elements(B*L*D)/s, 1 GPU" % ("fwd+bwd" if pair else "bwd"),
        "value": elems / (wall / args.steps), "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * wall / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == si.BF16 else "f32", "data": "synthetic (seeded)",
        "config": {"workload": w.name, "pass": args.which, "batch": w.batch, "L": w.L,
                   "dim": w.dim,
                   "N": w.N, "gate": w.gate,
                   "abar": "exp2_per_state" if general_a else "power_chain_s4d_real",
                   "keep_checkpoints": keep},
        "clock_ramp": {"calls": ramp[0], "ms": ramp[1]},
        "call_ms": {"mean": call_mean, "single_call_p50": float(np.median(call_ms)),
                    "timed_quarters": quarters},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": VALU_PEAK_SLOTS / 1e9,
                     "unit": "G VALU lane-slots/s", "frac": achieved * 1e9 / VALU_PEAK_SLOTS,
                     "traffic": None,
                     "kernel": ("selscan_fwd + selscan_bwd_ex (reusing the forward's part "
                                "state)" if pair else "selscan_bwd call (all passes)"),
                     "algorithmic_slots_per_element": slots_el,
                     "algorithmic_bytes_per_call": nb,
                     "hbm_gbps_of_call": nb / (call_mean * 1e-3) / 1e9},
    }
    if args.variant:
        res["variant"] = args.variant
        if not pair:
            res["roofline"]["kernel"] = "selscan_bwd_ex call (%s, all passes)" % args.variant
    print(json.dumps(res), flush=True)


def torch_loop_context(w, calls=2):
    """Context, not the product: the selective scan written as a plain PyTorch
    loop over timesteps on the GPU, the way the Mamba tutorial's section 4.2
    listing writes it (per step: A_bar = exp(Delta A), h = A_bar h + Delta B u,
    y = C.h, all as tensor ops; then D u and the SiLU(z) gate), in fp32, on
    the same inputs.  Returns the mean wall time per call and the ratio to
    selscan_fwd, which the pages' 20-40x claim is about."""
    import torch
    import torch.nn.functional as F

    import selective_state_space_selscan_amd as ss
    dev = torch.device("cuda:0")
    _, sets = make_inputs(w, dev, 1)
    t = sets[0]
    u, dl, z = (t[k].float() for k in ("u", "delta", "z"))
    Bm, Cm = t["Bm"].float(), t["Cm"].float()
    A, D, bias = t["A"], t["D_skip"], t["delta_bias"]

    def loop():
        dt = F.softplus(dl + bias)
        h = torch.zeros((w.batch, w.dim, w.N), dtype=torch.float32, device=dev)
        ys = []
        for s in range(w.L):
            dA = torch.exp(dt[:, s, :, None] * A)
            h = dA * h + (dt[:, s, :, None] * u[:, s, :, None]) * Bm[:, s, None, :]
            ys.append((h * Cm[:, s, None, :]).sum(-1))
        y = torch.stack(ys, 1) + D * u
        return y * F.silu(z)

    loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        loop()
    torch.cuda.synchronize()
    loop_ms = 1e3 * (time.perf_counter() - t0) / calls
    for _ in range(20):
        ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(50):
        ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, None)
    torch.cuda.synchronize()
    fwd_ms = 1e3 * (time.perf_counter() - t0) / 50
    return {"torch_loop_ms_per_call": loop_ms, "selscan_fwd_ms_per_call": fwd_ms,
            "speedup": loop_ms / fwd_ms, "calls": calls,
            "what": "plain PyTorch loop over the L timesteps on the GPU (fp32 tensor ops per "
                    "step), same inputs; context for the pages' 20-40x claim"}


VARIANT_FLAGS = {"zoh": 1, "rev": 2}


def parse_variant(spec):
    """'zoh,rev,conv4' -> (flags, conv width)."""
    flags, k = 0, 0
    for part in filter(None, (spec or "").split(",")):
        if part.startswith("conv"):
            k = int(part[4:] or 4)
        else:
            flags |= VARIANT_FLAGS[part]
    return flags, k


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before the timed ones")
    ap.add_argument("--ramp-ms", type=float, default=500.0,
                    help="untimed steps for this long (wall clock) before the warmup steps, so "
                         "that the clocks have ramped up (0: none); reported as clock_ramp")
    ap.add_argument("--workload", default="mamba130m_layer")
    ap.add_argument("--rotate", type=int, default=4, help="input-set copies to rotate")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--parse-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "fwdbwd"), default="fwd")
    ap.add_argument("--torch-loop", action="store_true",
                    help="context only: time a plain PyTorch loop over timesteps against "
                         "selscan_fwd on the workload, print one JSON line")
    ap.add_argument("--variant", default="", help="variants: zoh, rev, convK (fwd or bwd)")
    ap.add_argument("--keep-checkpoints", action="store_true",
                    help="--pass fwdbwd: the forward keeps the backward's checkpoints "
                         "(SELSCAN_FLAG_KEEP_CHECKPOINTS), the backward skips its checkpoint pass")
    ap.add_argument("--a", dest="a_form", choices=("s4d", "general"), default="s4d",
                    help="A = -(n+1) (S4D-real: the power-chain A_bar) or a perturbed, "
                         "general A (A_bar by one exp2 per (t, n))")
    args = ap.parse_args()

    import selscan_inputs as si
    w = si.WORKLOADS[args.workload]
    if args.parse_pmc:
        parse_pmc(w, *args.parse_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: one GPU only: the scan shards over (batch, dim) with no exchange, "
              "so throughput on several GPUs is not measured.", file=sys.stderr)
        sys.exit(2)
    if w.decode_steps:
        bench_decode(w, args.steps, args.warmup, args.ramp_ms)
        return
    if args.pmc_run:
        pmc_run(w, "bwd" if args.which == "bwd" else "fwd")
        return
    if args.torch_loop:
        print(json.dumps({"workload": w.name, **torch_loop_context(w)}), flush=True)
        return
    if args.which in ("bwd", "fwdbwd"):
        bench_bwd(w, args)
        return
    vflags, vconv = parse_variant(args.variant)

    import torch

    import selective_state_space_selscan_amd as ss

    dev = torch.device("cuda:0")
    inp, sets = make_inputs(w, dev, args.rotate)
    general_a = args.a_form == "general"
    if general_a:
        inp.A = si.perturbed_A(w.dim, w.N, w.seed)
        for t in sets:
            t["A"] = torch.from_numpy(inp.A).to(dev)
    es = 2 if w.dtype == si.BF16 else 4
    ys = [torch.empty((w.batch, w.L, w.dim), dtype=sets[0]["u"].dtype, device=dev)
          for _ in range(args.rotate)]
    hls = [torch.empty((w.batch, w.dim, w.N), dtype=torch.float32, device=dev)
           if w.want_last_state else None for _ in range(args.rotate)]
    code = ss.SELSCAN_BF16 if w.dtype == si.BF16 else ss.SELSCAN_F32
    ws_bytes = ss.selscan_fwd_workspace_bytes(w.batch, w.L, w.dim, w.N, code)
    wss = [torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
           for _ in range(args.rotate)]
    stream = torch.cuda.current_stream(dev)
    conv_w = conv_b = None
    if vconv:
        cw, cb = si.conv_params(w.dim, vconv, w.seed)
        conv_w, conv_b = torch.from_numpy(cw).to(dev), torch.from_numpy(cb).to(dev)

    def step(i):
        t = sets[i % args.rotate]
        if args.variant:
            ss.selscan_fwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                              t["delta_bias"], True, None, return_last_state=w.want_last_state,
                              flags=vflags, conv_weight=conv_w, conv_bias=conv_b,
                              y=ys[i % args.rotate], h_last=hls[i % args.rotate],
                              workspace=wss[i % args.rotate], stream=stream)
            return
        ss.selscan_fwd(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                       t["delta_bias"], True, None, return_last_state=w.want_last_state,
                       y=ys[i % args.rotate], h_last=hls[i % args.rotate],
                       workspace=wss[i % args.rotate], stream=stream)

    wall, call_mean, call_ms, quarters, ramp = timed_steps(step, args.steps, args.warmup, stream,
                                                             ramp_ms=args.ramp_ms)

    elems = w.batch * w.L * w.dim
    ms_per_step = 1e3 * wall / args.steps
    abytes = algorithmic_bytes(w.batch, w.L, w.dim, w.N, es, w.gate, w.want_last_state)
    slots_el = algorithmic_valu_slots(w.N, w.gate, es, general_a, vflags, vconv)
    slots = slots_el * elems
    achieved = slots / (call_mean * 1e-3) / 1e9
    peak = VALU_PEAK_SLOTS / 1e9
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
                   "gate": w.gate, "state": "fp32", "rotating_input_sets": args.rotate,
                   "A": ("general: -(n+1) exp(N(0, 0.25^2)) per (d, n)" if general_a
                         else "S4D-real: -(n+1)"),
                   "abar": "exp2_per_state" if general_a else "power_chain_s4d_real"},
        **({"variant": args.variant} if args.variant else {}),
        "hbm_gbps": abytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac": abytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "clock_ramp": {"calls": ramp[0], "ms": ramp[1]},
        "call_ms": {"mean": call_mean, "timed_quarters": quarters,
                    "single_call": {"p10": float(np.percentile(call_ms, 10)),
                                    "p50": float(np.median(call_ms)),
                                    "p90": float(np.percentile(call_ms, 90)),
                                    "calls": len(call_ms)}},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak,
                     "unit": "G VALU lane-slots/s", "frac": achieved / peak,
                     "traffic": None if general_a else load_traffic(w.name),
                     "kernel": "selscan_fwd call (summary, carry and main passes)",
                     "algorithmic_slots_per_element": slots_el,
                     "algorithmic_bytes_per_call": abytes,
                     "hbm_gbps_of_call": abytes / (call_mean * 1e-3) / 1e9,
                     "hbm_frac_of_call": abytes / (call_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS},
    }
    if args.variant:
        result["roofline"]["traffic"] = None
        result["roofline"]["kernel"] = "selscan_fwd_ex call (%s); slots of the default path" \
            % args.variant
    result["device_copy_gbps"] = device_copy_gbps(dev)
    if not args.no_cpu and not args.variant and not general_a:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
