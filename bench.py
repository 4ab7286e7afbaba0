"""Benchmark of the resolvent-head forward pass on one MI355X.

One step is one resolvent_forward call over the headline workload (B=4, H=16,
n=8192, d=128, bf16 q,k,v, switches (1,1,1)): the prologue (status clear, gates
and their in-tile products), the visit-count scan, the fused forward
kernel and the logit-overflow check, with the inputs already resident in HBM.
Prints one JSON line: the throughput, the per-stage times from HIP events, the
roofline object of the fused kernel and the oracle's CPU rate.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --workload {2,4,5} [--fp32]   # other workloads, one line per
                                                # switch setting; --fp32: the fp32 path
  python bench.py --path {chain,grouped,decode,operator}   # the other entry points
  python bench.py --copy-bytes N   # a plain copy kernel, for counter calibration
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "gated_causal_attention_amd", "csrc", "resolvent_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_pad_kernel_traffic_headline.json")
METRIC = "resolvent-head fwd TFLOP/s + Mtokens/s at n=8192,d=128; % bf16 MFMA peak"
FWD_KERNEL = "fwd_pad_kernel"  # the fused kernel of the bf16 path (rocprofv3 kernel-name filter)


def kernel_source_sha():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(sha):
    """HBM bytes per fused-kernel launch from the committed rocprofv3 counter
    runs, if they were taken on this exact kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration(nbytes):
    import torch

    a = torch.empty(nbytes // 4, device="cuda:0", dtype=torch.float32).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 3}), flush=True)


def counter_per_dispatch(run_dir, counter, name_filter):
    """Mean value of one rocprofv3 counter over the dispatches whose kernel name
    contains name_filter, from the CSV files under run_dir."""
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_filter in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_filter}' under {run_dir}")
    return sum(vals) / len(vals), len(vals)


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes):
    """HBM bytes per fused-kernel launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each divided by what the same counter reads per byte of a plain
    device copy of copy_bytes (torch copy_ of one device tensor into another: the
    runtime's copyBuffer kernel, which reads and writes copy_bytes)."""
    kf, nkf = counter_per_dispatch(fetch_dir, "FETCH_SIZE", FWD_KERNEL)
    kw, nkw = counter_per_dispatch(write_dir, "WRITE_SIZE", FWD_KERNEL)
    cf, _ = counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _ = counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f_fac = cf * 1024.0 / copy_bytes
    w_fac = cw * 1024.0 / copy_bytes
    fetch = kf * 1024.0 / f_fac
    write = kw * 1024.0 / w_fac
    return {
        "kernel": "fwd_pad_kernel<d=128, dv=128> (headline workload, switches (1,1,1))",
        "kernel_source_sha256": kernel_source_sha(),
        "fetch_size_kib_per_dispatch": kf, "write_size_kib_per_dispatch": kw,
        "dispatches": [nkf, nkw],
        "copy_bytes": copy_bytes,
        "copy_fetch_size_kib": cf, "copy_write_size_kib": cw,
        "fetch_factor": f_fac, "write_factor": w_fac,
        "hbm_read_bytes_per_launch": fetch, "hbm_write_bytes_per_launch": write,
        "traffic_bytes_per_launch": fetch + write,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -d F -o run --output-format csv -- python3 bench.py "
            "--steps 2 --warmup 1 --no-cpu-baseline",
            "rocprofv3 --pmc WRITE_SIZE -d W -o run --output-format csv -- python3 bench.py "
            "--steps 2 --warmup 1 --no-cpu-baseline",
            f"rocprofv3 --pmc FETCH_SIZE -d CF -o run --output-format csv -- python3 bench.py "
            f"--copy-bytes {copy_bytes}",
            f"rocprofv3 --pmc WRITE_SIZE -d CW -o run --output-format csv -- python3 bench.py "
            f"--copy-bytes {copy_bytes}",
            f"python3 bench.py --summarize-traffic F W CF CW --copy-bytes {copy_bytes}"],
    }


COUNTER_FILE = os.path.join(ROOT, "profiles", "fwd_pad_kernel_counters_headline.json")
# rocprofv3 --pmc passes over the headline bench (each within one pass's
# hardware limits: at most 8 SQ_, 4 TCC_ and 2 GRBM_ counters)
COUNTER_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_SALU "
    "SQ_INSTS_LDS SQ_WAVES GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES "
    "SQ_WAIT_INST_LDS SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT TCC_HIT_sum TCC_MISS_sum "
    "GRBM_GUI_ACTIVE",
)
SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs
XCDS = 8


def summarize_counters(dirs):
    """Utilisation figures of the fused kernel from the COUNTER_PASSES runs
    (one directory per pass, in order).  Every counter is the mean per
    dispatch of fwd_kernel; the SQ_ counters are summed over the chip by
    rocprofv3, and GRBM_GUI_ACTIVE (active cycles) is summed over the 8 XCDs,
    so the GPU's active cycles during the dispatch are GRBM_GUI_ACTIVE / 8.
      mfma_busy_pct   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs)
      mfma_coexec_pct = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES
                        (share of the matrix-busy cycles in which a vector
                        instruction also issued on the SIMD)
      mfma_flops      = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
      valu_per_mfma   = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA
                        (SQ_INSTS_VALU counts the MFMAs too)
      lds_bank_conflict_pct = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      l2_hit_pct      = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)"""
    vals = {}
    for d, names in zip(dirs, COUNTER_PASSES):
        for c in names.split():
            vals.setdefault(c, counter_per_dispatch(d, c, FWD_KERNEL)[0])
    busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"]
    gui = vals["GRBM_GUI_ACTIVE"]
    out = {
        "kernel": "fwd_pad_kernel<d=128, dv=128> (headline workload, switches (1,1,1))",
        "kernel_source_sha256": kernel_source_sha(),
        "counters_per_dispatch": vals,
        "mfma_busy_pct": 100.0 * busy / (gui / XCDS * SIMDS),
        "active_cycles": gui / XCDS,
        "mfma_coexec_pct": 100.0 * vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy,
        "mfma_flops_per_dispatch": vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
        "valu_per_mfma": (vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / vals["SQ_INSTS_MFMA"],
        "salu_per_mfma": vals["SQ_INSTS_SALU"] / vals["SQ_INSTS_MFMA"],
        "lds_per_mfma": vals["SQ_INSTS_LDS"] / vals["SQ_INSTS_MFMA"],
        "lds_bank_conflict_pct": 100.0 * vals["SQ_LDS_BANK_CONFLICT"] / vals["SQ_LDS_IDX_ACTIVE"],
        "l2_hit_pct": 100.0 * vals["TCC_HIT_sum"] / (vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"]),
        "derivation": summarize_counters.__doc__.split("\n", 5)[5].strip(),
        "commands": [f"rocprofv3 --pmc {p} -d P{i} -o run --output-format csv -- python3 "
                     f"bench.py --steps 2 --warmup 1 --no-cpu-baseline"
                     for i, p in enumerate(COUNTER_PASSES)] +
                    ["python3 bench.py --summarize-counters P0 P1 P2"],
    }
    return out


def measured_counters(sha):
    """The utilisation summary of the committed counter runs, if they were
    taken on this exact kernel source; else None."""
    try:
        with open(COUNTER_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    keys = ("mfma_busy_pct", "mfma_coexec_pct", "mfma_flops_per_dispatch", "valu_per_mfma",
            "salu_per_mfma", "lds_per_mfma", "lds_bank_conflict_pct", "l2_hit_pct")
    return {k: rec[k] for k in keys}


def cpu_baseline(inp, sw, heads, rows=None, flops_per_pair=None):
    """The fp64 oracle, as it stands, on the given heads (all rows, or the given
    rows) of the same inputs; FLOPs are counted dense-causal: row i has i+1
    pairs of flops_per_pair (default 6 d) each."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    n, d = inp["n"], inp["d"]
    if flops_per_pair is None:
        flops_per_pair = 6 * d
    all_rows = rows is None
    if all_rows:
        rows = np.arange(n)
    t0 = time.perf_counter()
    for b, h in heads:
        st, _ = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h], inp["u"][b, h],
                                    inp["theta"][b, h], inp["v"][b, h], *sw, rows=rows,
                                    nthreads=threads)
        assert st == oracle.OK
    dt = time.perf_counter() - t0
    flops = float(flops_per_pair) * float(np.sum(rows + 1)) * len(heads)
    what = (f"all {n} rows" if all_rows
            else f"{len(rows)} of {n} rows (every {rows[1] - rows[0]}th from {rows[0]})")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(heads)} heads (b,h) = {heads} of the same workload, {what}, "
                      f"fp64; {dt:.2f} s; FLOPs counted dense-causal ({flops_per_pair} per "
                      f"(query, key) pair, i+1 pairs in row i)",
            "cpu_model": cpu_model(),
            "seconds": dt, "head_tokens_per_s": len(heads) * len(rows) / dt}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def chain_cpu_baseline(inp, g, heads):
    """The oracle's gated chain, as it stands, on whole heads of the same inputs."""
    import numpy as np

    import oracle

    dv = inp["v"].shape[-1]
    n = inp["n"]
    t0 = time.perf_counter()
    for b, h in heads:
        st, a = oracle.gates(inp["u"][b, h], inp["theta"][b, h], g)
        assert st == oracle.OK
        for c in range(dv):
            oracle.chain(a, inp["v"][b, h, :, c], y0_from_b0=True)
    dt = time.perf_counter() - t0
    nbytes = len(heads) * n * (8 + 2 * dv + 8 * dv)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(heads)} whole heads of the same inputs, all {dv} channels, fp64, "
                      f"one thread; {dt:.2f} s; bytes counted as on the device (u, theta, "
                      f"bf16 v in, fp32 O out)",
            "seconds": dt}


def bench_chain(args):
    """The chain-corner scan (resolvent_chain) on the headline inputs."""
    import numpy as np
    import torch

    from gated_causal_attention_amd import binding, inputs

    dev = torch.device("cuda:0")
    g = 1.0
    inp = inputs.make_config(3)
    B, H, n = inp["B"], inp["H"], inp["n"]
    dv = inp["v"].shape[-1]
    t = inputs.as_torch(inp, dev)
    o_re = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    o_im = torch.empty_like(o_re)
    ws = torch.empty(binding.resolvent_chain_workspace_bytes(B, H, n, dv), device=dev,
                     dtype=torch.uint8)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.resolvent_chain(t["u"], t["theta"], t["v"], g, o_re=o_re, o_im=o_im,
                                workspace=ws, status=status, stream=stream, check=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ms_per_step = start.elapsed_time(end) / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # algorithmic HBM bytes: u, theta in; bf16 v in; O_re, O_im out
    alg = B * H * n * (8 + 2 * dv + 8 * dv)
    achieved = alg / (call_ms * 1e-3) / 1e9
    out = {
        "metric": "chain-corner scan (resolvent_chain): GB/s of algorithmic HBM traffic",
        "value": alg / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "chain corner O_i = sum_j G_ij V_j at g = 1 on the headline "
                               "inputs: B=4 H=16 n=8192 dv=128, bf16 v ~ N(0,1), "
                               "u ~ U(0.95,1), theta ~ U(-0.05,0.05), seed 3",
                   "B": B, "H": H, "n": n, "dv": dv, "g": g},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "resolvent_chain (gates + three scan kernels, one call)",
                     "bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = chain_cpu_baseline(inp, g, [(0, 0), (1, 5), (2, 10), (3, 15)])
    print(json.dumps(out), flush=True)


def bench_grouped(args):
    """resolvent_forward_grouped on a grouped workload: 16 query heads sharing
    2 k/v heads per batch entry, value width 64."""
    import numpy as np
    import torch

    from gated_causal_attention_amd import binding, inputs

    dev = torch.device("cuda:0")
    sw = (1, 1, 1)
    B, H, Hkv, n, d, dv = 4, 16, 2, 8192, 128, 64
    inp = inputs.draw(B, H, n, d, 7, dv=dv, u_range=(0.95, 1.0), theta_range=(-0.05, 0.05))
    inp["k"] = np.ascontiguousarray(inp["k"][:, :Hkv])
    inp["v"] = np.ascontiguousarray(inp["v"][:, :Hkv])
    t = inputs.as_torch(inp, dev)
    o_re = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    o_im = torch.empty_like(o_re)
    ws = torch.empty(binding.resolvent_workspace_bytes_grouped(B, H, Hkv, n, d, dv), device=dev,
                     dtype=torch.uint8)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream = torch.cuda.current_stream(dev)
    cnt_off = binding.resolvent_counters_offset(B, H, n, d)

    def step():
        binding.resolvent_forward_grouped(t["q"], t["k"], t["u"], t["theta"], t["v"], *sw,
                                          o_re=o_re, o_im=o_im, workspace=ws, status=status,
                                          stream=stream, check=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ms_per_step = start.elapsed_time(end) / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    BQ, BK = binding.resolvent_tile_shape()
    off_tiles = int(ws[cnt_off:cnt_off + 4].cpu().numpy().view(np.uint32)[0])
    n_qt = (n + BQ - 1) // BQ
    diag_pairs = B * H * sum(min(BQ, n - q * BQ) * (min(BQ, n - q * BQ) + 1) // 2
                             for q in range(n_qt))
    eval_pairs = off_tiles * BQ * BK + diag_pairs
    alg_flops = (2 * d + 4 * dv) * eval_pairs
    achieved = alg_flops / (call_ms * 1e-3) / 1e12
    out = {
        "metric": "grouped resolvent head (resolvent_forward_grouped): TFLOP/s",
        "value": alg_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "grouped head B=4 H=16 Hkv=2 n=8192 d=128 dv=64, bf16 q,k,v "
                               "~ N(0,1), u ~ U(0.95,1), theta ~ U(-0.05,0.05), switches "
                               "(1,1,1), seed 7",
                   "B": B, "H": H, "Hkv": Hkv, "n": n, "d": d, "dv": dv},
        "mtokens_per_s": B * n / (ms_per_step * 1e-3) / 1e6,
        "evaluated_pair_fraction": eval_pairs * 2.0 / (n * (n + 1) * B * H),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "resolvent_forward_grouped (whole call)",
                     "flops_per_launch": alg_flops},
    }
    if not args.no_cpu_baseline:
        heads = [(0, 0), (1, 9)]
        import oracle

        t0 = time.perf_counter()
        for b, h in heads:
            st, _ = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h // (H // Hkv)],
                                        inp["u"][b, h], inp["theta"][b, h],
                                        inp["v"][b, h // (H // Hkv)], *sw, rows=np.arange(n),
                                        nthreads=oracle.default_threads())
            assert st == oracle.OK
        dt = time.perf_counter() - t0
        flops = (d + 2 * dv) * n * (n + 1) * len(heads)
        out["cpu_baseline"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.default_threads(), "kind": "oracle",
                               "cpu_model": cpu_model(),
                               "sample": f"{len(heads)} whole heads {heads}, all {n} rows, fp64; "
                                         f"{dt:.2f} s; FLOPs counted dense-causal"}
    print(json.dumps(out), flush=True)


def bench_decode(args):
    """One decode step (resolvent_decode) on the headline inputs: the readout
    of position n-1 of every head against caches of n = 8192 positions."""
    import numpy as np
    import torch

    from gated_causal_attention_amd import binding, inputs

    dev = torch.device("cuda:0")
    sw = (1, 1, 1)
    inp = inputs.make_config(3)
    B, H, n, d = inp["B"], inp["H"], inp["n"], inp["d"]
    dv = inp["v"].shape[-1]
    t = inputs.as_torch(inp, dev)
    q = t["q"][:, :, n - 1].contiguous()
    o_re = torch.empty((B, H, dv), device=dev, dtype=torch.float32)
    o_im = torch.empty_like(o_re)
    ws = torch.empty(binding.resolvent_decode_workspace_bytes(B, H, H, n, d, dv), device=dev,
                     dtype=torch.uint8)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.resolvent_decode(q, t["k"], t["u"], t["theta"], t["v"], *sw, o_re=o_re,
                                 o_im=o_im, workspace=ws, status=status, stream=stream,
                                 check=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ms_per_step = start.elapsed_time(end) / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # algorithmic HBM bytes of a step: the bf16 caches k, v and the fp32 u, theta
    # of n positions, the query in, the complex fp32 readout out
    per_head = n * (2 * d + 2 * dv + 8) + 2 * d + 8 * dv
    alg = B * H * per_head
    achieved = alg / (call_ms * 1e-3) / 1e9
    out = {
        "metric": "decode step (resolvent_decode): GB/s of algorithmic HBM traffic",
        "value": alg / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode step: the readout of position n-1 of every head, "
                               "headline inputs B=4 H=16 n=8192 d=128 dv=128, bf16 q,k,v "
                               "~ N(0,1), u ~ U(0.95,1), theta ~ U(-0.05,0.05), switches "
                               "(1,1,1), seed 3, query = q[:, :, n-1]",
                   "B": B, "H": H, "n": n, "d": d, "dv": dv},
        "decode_steps_per_s": 1e3 / ms_per_step,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "resolvent_decode (part and merge kernels: one call)",
                     "bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        import oracle

        heads = [(b, h) for b in range(B) for h in range(H)]
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < 10.0 and done < 40 * len(heads):
            b, h = heads[done % len(heads)]
            st, _ = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h], inp["u"][b, h],
                                        inp["theta"][b, h], inp["v"][b, h], *sw,
                                        rows=[n - 1], nthreads=1)
            assert st == oracle.OK
            done += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done * per_head / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"{done} head decode steps (row n-1 of the same "
                                         f"heads, cycled), fp64, one thread; {dt:.2f} s; "
                                         f"bytes counted as on the device"}
    print(json.dumps(out), flush=True)


def bench_operator(args):
    """The materialising exports at a small-n workload: resolvent_operator
    writing W [B,H,n,n] (float32) and resolvent_path_product writing G (f64)
    for the same heads' gates."""
    import numpy as np
    import torch

    from gated_causal_attention_amd import binding, inputs

    dev = torch.device("cuda:0")
    sw = (1, 1, 1)
    B, H, n, d = 1, 16, 2048, 128
    inp = inputs.draw(B, H, n, d, 11, u_range=(0.95, 1.0), theta_range=(-0.05, 0.05))
    t = inputs.as_torch(inp, dev)
    w_re = torch.empty((B, H, n, n), device=dev, dtype=torch.float32)
    w_im = torch.empty_like(w_re)
    ws = torch.empty(binding.resolvent_operator_workspace_bytes(B, H, n, d), device=dev,
                     dtype=torch.uint8)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream = torch.cuda.current_stream(dev)
    gre, gim = inputs.draw_complex_gates(H, n, 12)
    a_re = torch.from_numpy(gre).to(dev)
    a_im = torch.from_numpy(gim).to(dev)
    g_re = torch.empty((H, n, n), device=dev, dtype=torch.float64)
    g_im = torch.empty_like(g_re)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for x, y in ev:
            x.record(stream)
            fn()
            y.record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        return (start.elapsed_time(end) / args.steps,
                float(np.mean([x.elapsed_time(y) for x, y in ev])))

    ms_op, call_op = timed(lambda: binding.resolvent_operator(
        t["q"], t["k"], t["u"], t["theta"], *sw, w_re=w_re, w_im=w_im, workspace=ws,
        status=status, stream=stream, check=False))
    assert int(status.item()) == 0
    ms_pp, _ = timed(lambda: binding.resolvent_path_product(a_re, a_im, g_re=g_re, g_im=g_im,
                                                            stream=stream))
    # algorithmic HBM bytes: q, k, u, theta in; W out (float32 complex, n^2 per head)
    alg = B * H * (2 * n * d * 2 + 8 * n + 8 * n * n)
    achieved = alg / (call_op * 1e-3) / 1e9
    out = {
        "metric": "operator export (resolvent_operator): GB/s of algorithmic HBM traffic",
        "value": alg / (ms_op * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_op,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "operator W of B=1 H=16 heads at n=2048 d=128, bf16 q,k "
                               "~ N(0,1), u ~ U(0.95,1), theta ~ U(-0.05,0.05), switches "
                               "(1,1,1), seed 11; path_product of 16 rows of n gates "
                               "r e^{i phi}, r ~ U(0.95,1), phi ~ U(-0.05,0.05), seed 12",
                   "B": B, "H": H, "n": n, "d": d},
        "path_product_ms": ms_pp,
        "path_product_gbs": H * n * n * 16 / (ms_pp * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "resolvent_operator (gates + block kernels: one call)",
                     "bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        import oracle

        heads = [0, 9]
        t0 = time.perf_counter()
        for h in heads:
            st, _ = oracle.operator(inp["q"][0, h], inp["k"][0, h], inp["u"][0, h],
                                    inp["theta"][0, h], *sw)
            assert st == oracle.OK
        dt = time.perf_counter() - t0
        per_head = 2 * n * d * 2 + 8 * n + 8 * n * n
        out["cpu_baseline"] = {"value": len(heads) * per_head / dt / 1e9, "unit": "GB/s",
                               "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"the oracle's operator on heads {heads}, fp64, one "
                                         f"thread; {dt:.2f} s; bytes counted as on the device"}
    print(json.dumps(out), flush=True)


PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA


def _workload_inputs(widx, fp32):
    """The seeded inputs of workload widx; with fp32 the same draw (seed, shape,
    distributions) in fp32 q, k, v storage, for the fp32 MFMA path."""
    from gated_causal_attention_amd import inputs

    if not fp32:
        return inputs.make_config(widx)
    w = inputs.WORKLOADS[widx]
    return inputs.draw(w.B, w.H, w.n, w.d, widx, inputs.F32, inputs.F32, w.qk_scale, w.gates,
                       w.u_range, w.theta_range)


def _describe(inp, widx, sw, fp32):
    from gated_causal_attention_amd import inputs

    w = inputs.WORKLOADS[widx]
    dt = "fp32 q,k,v" if fp32 else f"{w.qk_dtype} q,k, {w.v_dtype} v"
    if w.gates == "bedm":
        gates = "gates in {-1,0,+1} with p = (0.05, 0.01, 0.94)"
    elif w.theta_range[0] == w.theta_range[1]:
        gates = f"u ~ U{tuple(w.u_range)}, theta = {w.theta_range[0]}"
    else:
        gates = (f"u ~ U{tuple(w.u_range)}, theta ~ U({w.theta_range[0]:.3g},"
                 f"{w.theta_range[1]:.3g})")
    scale = "" if w.qk_scale == 1.0 else f", q,k scaled by {w.qk_scale}"
    return (f"resolvent head B={inp['B']} H={inp['H']} n={inp['n']} d={inp['d']}, {dt} "
            f"~ N(0,1){scale}, {gates}, switches {tuple(sw)}, seed {widx}")


def forward_line(args, widx, sw, fp32, headline, inp=None):
    """Time resolvent_forward on workload widx at switches sw and print one JSON
    line: throughput, stage times from HIP events on the call's stream, the
    fused kernel's roofline (matrix or HBM bound, whichever its algorithmic
    work puts first at peak) and the oracle's CPU rate on a bounded sample."""
    import numpy as np
    import torch

    from gated_causal_attention_amd import binding, inputs

    dev = torch.device("cuda:0")
    if inp is None:
        inp = _workload_inputs(widx, fp32)
    B, H, n, d = inp["B"], inp["H"], inp["n"], inp["d"]
    dv = inp["v"].shape[-1]
    qdt = binding.F32 if inp["qk_dtype"] == inputs.F32 else binding.BF16
    vdt = binding.F32 if inp["v_dtype"] == inputs.F32 else binding.BF16
    t = inputs.as_torch(inp, dev)
    o_re = torch.empty((B, H, n, d), device=dev, dtype=torch.float32)
    o_im = torch.empty_like(o_re)
    ws_bytes = binding.resolvent_workspace_bytes(B, H, n, d, qdt, vdt)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream = torch.cuda.current_stream(dev)
    cnt_off = binding.resolvent_counters_offset(B, H, n, d, qdt, vdt)

    def step(marks=None):
        binding.resolvent_forward(t["q"], t["k"], t["u"], t["theta"], t["v"], *sw, o_re=o_re,
                                  o_im=o_im, workspace=ws, status=status, stream=stream,
                                  check=False, marks=marks)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, binding.resolvent_status_str(int(status.item()))

    K = args.steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for ms in marks:  # materialise the HIP events before they are handed to the library
        for e in ms:
            e.record(stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step([e.cuda_event for e in marks[i]])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    st = int(status.item())
    assert st == 0, binding.resolvent_status_str(st)
    fwd_ms = [m[1].elapsed_time(m[2]) for m in marks]
    pre_ms = [m[0].elapsed_time(m[1]) for m in marks]
    post_ms = [m[2].elapsed_time(m[3]) for m in marks]
    fwd_avg = float(np.mean(fwd_ms))
    ms_per_step = total_ms / K

    # work: (query, key) pairs the fused kernel evaluated in one launch
    BQ, BK = binding.resolvent_tile_shape()
    off_tiles = int(ws[cnt_off:cnt_off + 4].cpu().numpy().view(np.uint32)[0])
    n_qt = (n + BQ - 1) // BQ
    diag_pairs = B * H * sum(min(BQ, n - q * BQ) * (min(BQ, n - q * BQ) + 1) // 2
                             for q in range(n_qt))
    eval_pairs = off_tiles * BQ * BK + diag_pairs
    # 2d for the logit (none at qk = 0, where the logit matrix is skipped) and
    # 4 dv for the complex readout (two real-by-real products)
    flops_per_pair = (2 * d if sw[1] != 0 else 0) + 4 * dv
    alg_flops = flops_per_pair * eval_pairs
    dense_flops = (flops_per_pair / 2.0) * n * (n + 1) * B * H
    nw = BQ // 32  # waves per query tile; wave w runs w+1 blocks of 32x32 on the diagonal
    diag_blocks_exec = B * H * n_qt * (nw * (nw + 1) // 2)
    exec_flops = flops_per_pair * (off_tiles * BQ * BK + diag_blocks_exec * 32 * 32)
    # HBM bytes the problem moves once: q, k, v and u, theta in; O_re, O_im out
    esz = {inputs.F32: 4, inputs.BF16: 2}
    alg_bytes = B * H * n * (2 * d * esz[inp["qk_dtype"]] + dv * esz[inp["v_dtype"]] + 8
                             + 8 * dv)
    peak_flops = PEAK_FP32_MFMA_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    mfma_bound = alg_flops / (peak_flops * 1e12) >= alg_bytes / (PEAK_HBM_GBS * 1e9)
    kname = (f"fwd_kernel<fp32, d={d}, dv={dv}>" if fp32
             else f"fwd_pad_kernel<d={d}, dv={dv}{', qk=0' if sw[1] == 0 else ''}>")
    if mfma_bound:
        achieved = alg_flops / (fwd_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_flops, "unit": "TFLOP/s",
                "frac": achieved / peak_flops}
    else:
        achieved = alg_bytes / (fwd_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    sha = kernel_source_sha()
    roof.update({"traffic": measured_traffic(sha) if headline else None, "kernel": kname,
                 "flops_per_launch": alg_flops, "bytes_per_launch": alg_bytes,
                 "executed_mfma_flops": exec_flops,
                 "executed_mfma_tflops": exec_flops / (fwd_avg * 1e-3) / 1e12})
    if headline:
        roof["counters"] = measured_counters(sha)
    out = {
        "metric": METRIC,
        "value": alg_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": _describe(inp, widx, sw, fp32), "B": B, "H": H, "n": n, "d": d,
                   "switches": list(sw)},
        "mtokens_per_s": B * n / (ms_per_step * 1e-3) / 1e6,
        "head_mtokens_per_s": B * H * n / (ms_per_step * 1e-3) / 1e6,
        "hbm_gbs_whole_call": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "pct_mfma_peak": 100.0 * alg_flops / (fwd_avg * 1e-3) / 1e12 / peak_flops,
        "dense_causal_equiv_tflops": dense_flops / (ms_per_step * 1e-3) / 1e12,
        "evaluated_pair_fraction": eval_pairs * 2.0 / (n * (n + 1) * B * H),
        "stage_ms": {"prologue": float(np.mean(pre_ms)), "fwd_kernel": fwd_avg,
                     "logit_check": float(np.mean(post_ms))},
        "roofline": roof,
    }
    if headline:
        out["pct_bf16_mfma_peak"] = out["pct_mfma_peak"]
    if not args.no_cpu_baseline:
        heads, rows = _cpu_sample(widx, B, H, n)
        out["cpu_baseline"] = cpu_baseline(inp, sw, heads, rows, flops_per_pair)
    print(json.dumps(out), flush=True)


def _cpu_sample(widx, B, H, n):
    """Heads (and rows) of a workload that the oracle finishes in ~5-30 s."""
    import numpy as np

    if widx == 3:
        return [(b, h) for b in range(B) for h in range(0, H, 2)], None  # half the 64 heads
    if widx == 4:  # one head of n = 32768: every 4th row (row i costs O(i d))
        return [(0, 0)], np.arange(3, n, 4)
    if widx == 5:  # 15 of the 256 heads
        return [(b, 0) for b in range(B)] + [(0, h) for h in range(1, 8)], None
    return [(b, h) for b in range(B) for h in range(H)], None


def bench_workload(args):
    """--workload W [--fp32]: one JSON line per switch setting of workload W."""
    from gated_causal_attention_amd import inputs

    widx = args.workload
    inp = _workload_inputs(widx, args.fp32)
    for sw in inputs.WORKLOADS[widx].switches:
        forward_line(args, widx, sw, args.fp32, headline=False, inp=inp)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--path", choices=("forward", "chain", "grouped", "decode", "operator"),
                    default="forward",
                    help="forward: the head (the headline line); chain: the chain-corner "
                         "scan; grouped: shared k/v heads and another value width; decode: "
                         "one decode step against an n-position cache; operator: the "
                         "materialising exports")
    ap.add_argument("--workload", type=int, choices=(2, 3, 4, 5), default=3,
                    help="forward path on another workload's shape, distributions and "
                         "switch settings (one line per setting); 3 is the headline")
    ap.add_argument("--fp32", action="store_true",
                    help="forward path with fp32 q, k, v (the fp32 MFMA path)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                              "COPY_WRITE"))
    ap.add_argument("--summarize-counters", nargs=len(COUNTER_PASSES),
                    metavar=tuple(f"PASS{i}" for i in range(len(COUNTER_PASSES))))
    args = ap.parse_args()
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(*args.summarize_traffic, args.copy_bytes), indent=1))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the resolvent head's heads are independent and the "
              "library has no multi-GPU path (a sharded run would split the (batch, head) "
              "pairs over the GPUs); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_bytes:  # the calibration copy of the traffic counters
        copy_calibration(args.copy_bytes)
        return

    if args.path == "chain":
        bench_chain(args)
        return
    if args.path == "grouped":
        bench_grouped(args)
        return
    if args.path == "decode":
        bench_decode(args)
        return
    if args.path == "operator":
        bench_operator(args)
        return

    if args.workload != 3 or args.fp32:
        bench_workload(args)
        return
    forward_line(args, 3, (1, 1, 1), fp32=False, headline=True)


if __name__ == "__main__":
    main()
