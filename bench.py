"""Throughput of one CP rank's share of causal THD attention on one MI355X.

A step is one pass of the whole hot path over the configured rank shares of
the Llama-3-8B-shaped packed workload (T = 32768 bf16 tokens, 32 q / 8 kv
heads, head dim 128, log-normal document lengths padded to multiples of 8,
cp_size = 4, ranks 0 and 3, both strategies).  For every share:

  partition indices -> (DualChunkSwap: K/V restoration from the rank-major
  gathered buffer) -> attention plan -> forward (O, LSE) -> backward (dQ, dK, dV)

Inputs are resident in HBM before the timed region.  The metric is useful
causal attention FLOP/s: forward 4*D*Hq*N, backward 10*D*Hq*N, with N the
number of (query, key) pairs the causal document mask allows for the share's
actual query rows.  Extra legs (skipped with --no-allgathered, as in profiling
runs), reported under breakdown:
  allgathered_path          the same shares with attention reading the
                            rank-major gathered K/V directly (no restoration);
  graph_replayed_step       the main step replayed from a HIP graph;
  partition_million_tokens  the partition kernel alone at T = 1,048,576 in
                            10,000 documents, every rank and strategy;
  dynamic_t_sweep           every share of 16 micro-batches of varying active T
                            on buffers allocated once for 65,536 tokens;
  long_context_shares       contiguous ranks 0 and 7 of the 70B-shaped
                            T = 131,072 workload (64 q / 8 kv heads, cp_size 8);
  short_mha_forward         the forward-only T = 8,192 workload (16 q / 16 kv
                            heads, cp_size 2), both strategies, ranks 0 and 1.
Prints one JSON line; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
SHARES = [(0, 0), (0, 3), (1, 0), (1, 3)]   # (strategy, rank)
STRAT_NAME = {0: "dcs", 1: "contiguous"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_t32768_gqa32x8_hbm_traffic.json")
KERNEL_SOURCES = ("attn_bwd.hip", "attn_fwd.hip", "attn_common.h", "cpthd_device.h")
# the physical-order kernels the main step launches at head_dim 128 (rocprofv3 kernel names)
KERNEL_SYMBOL = {"attn_fwd": "cpthd::attn_fwd_kernel<128, 1, false>",
                 "attn_bwd_dq": "cpthd::attn_bwd_dq_kernel<128, 1, false>",
                 "attn_bwd_dkdv": "cpthd::attn_bwd_dkdv_kernel<128, 2, false>"}


def kernel_source_hash(root=ROOT):
    """sha256 of the attention kernels' code: the sources with comments removed and whitespace collapsed, so a
    comment edit does not invalidate counters taken on the same code."""
    import hashlib
    import re
    code = []
    for f in KERNEL_SOURCES:
        text = open(os.path.join(root, "context_causal_thd_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        code.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    calibrated on a plain copy), or None when the kernel sources changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if kernel_source_hash() != rec.get("source_sha256"):
        return None
    v = rec["kernels"].get(KERNEL_SYMBOL[kernel])
    return None if v is None else v["fetch_bytes_per_launch"] + v["write_bytes_per_launch"]


class ClockSampler:
    """Samples the GPU shader clock (the starred level of the amdgpu kernel driver's pp_dpm_sclk file) every 2 ms from a
    background thread while the timed steps run; reads a file, starts nothing."""

    def __init__(self):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        while not self._stop.is_set():
            for path in self.paths:
                try:
                    for line in open(path):
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*Mhz", line, flags=re.I)
                            if m:
                                self.samples.append(int(m.group(1)))
                except OSError:
                    return
            time.sleep(0.002)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        return {"median_mhz": float(np.median(self.samples)), "min_mhz": int(min(self.samples)),
                "samples": len(self.samples), "source": "pp_dpm_sclk current level, sampled every 2 ms"}


def useful_pairs(idx, cu_p, cu_a):
    """Allowed (query, key) pairs for the rank's query rows: sum over actual rows of (position + 1)."""
    cu_p = cu_p.astype(np.int64)
    cu_a = cu_a.astype(np.int64)
    doc = np.searchsorted(cu_p, idx, side="right") - 1
    pos = idx - cu_p[doc]
    actual = cu_a[doc + 1] - cu_a[doc]
    ok = pos < actual
    return int(np.sum(pos[ok] + 1))


def cpu_baseline(wl, budget_s=15.0):
    """Time the CPU oracle (fwd + bwd) on a bounded sample: whole kv heads of the DualChunkSwap rank-0 share."""
    import oracle
    from threadpoolctl import threadpool_info

    idx = oracle.partition_indices(wl.cu_padded, wl.cp, 0, 0)
    q, k, v, do = wl.q(idx), wl.k(), wl.v(), wl.do(idx)
    pairs = useful_pairs(idx, wl.cu_padded, wl.cu_actual)
    G = wl.Hq // wl.Hkv
    t0 = time.perf_counter()
    heads = 0
    for g in range(wl.Hkv):
        oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, kv_heads=[g])
        oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, kv_heads=[g])
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 14.0 * wl.D * G * heads * pairs
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd+bwd of {heads} of {wl.Hkv} kv heads ({heads * G} of {wl.Hq} q heads) of the "
                      f"DualChunkSwap rank-0 share, all {wl.num_docs} documents ({pairs} causal pairs per head), "
                      f"float64 numpy, {dt:.1f} s"}


def dynamic_t_sweep(cpthd, torch, dev, status, reps=3):
    """The dynamic-T micro-batch sweep on buffers allocated once for 65,536 tokens: 16 micro-batches whose active
    T varies (multiples of 64 in [4096, 65536]), cp_size 4, both strategies, every rank; each share runs the
    full step (partition, restoration under DualChunkSwap, plan, forward, backward) on the active prefix.  Per
    micro-batch the eight shares' inputs are staged first, then the eight steps run back-to-back between two
    events (reps times, after one untimed pass).  Tensor values are drawn on the GPU (timing only)."""
    cap, cp = W.DYNAMIC_T_CAPACITY, 4
    Hq, Hkv, D = 32, 8, 128
    scale = 1.0 / math.sqrt(D)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def randn(shape, sd):
        return (torch.randn(shape, generator=gen, device=dev) * sd).to(torch.bfloat16)

    k_phys, v_phys = randn((cap, Hkv, D), 0.5), randn((cap, Hkv, D), 0.5)
    q_full, do_full = randn((cap, Hq, D), 0.5), randn((cap, Hq, D), 1.0)
    capS = cap // cp
    kg, vg = torch.empty_like(k_phys), torch.empty_like(v_phys)
    k_buf, v_buf = torch.empty_like(k_phys), torch.empty_like(v_phys)
    o = torch.empty((capS, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((capS, Hq), dtype=torch.float32, device=dev)
    dq = torch.empty((capS, Hq, D), dtype=torch.float32, device=dev)
    dk = torch.empty((cap, Hkv, D), dtype=torch.float32, device=dev)
    dv = torch.empty((cap, Hkv, D), dtype=torch.float32, device=dev)
    idx_out = torch.empty(capS, dtype=torch.int32, device=dev)
    layouts = [W.dynamic_t(m) for m in range(W.DYNAMIC_T_MICROBATCHES)]
    plan = cpthd.AttnPlan(cap, cp, Hq, Hkv, D, max_docs=max(wl.num_docs for wl in layouts))
    q_loc = [torch.empty((capS, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(cp)]
    do_loc = [torch.empty((capS, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(cp)]
    total_ms, flops = 0.0, {0: 0.0, 1: 0.0}
    ms_by_strategy = {0: 0.0, 1: 0.0}
    for wl in layouts:
        T, S = wl.T, wl.T // cp
        cu_a = torch.from_numpy(wl.cu_actual).to(dev)
        cu_p = torch.from_numpy(wl.cu_padded).to(dev)
        for s in (0, 1):
            # staging (untimed): the ranks' local Q / dO rows and, under DualChunkSwap, the rank-major gathered K/V
            parts = [cpthd.partition_indices(cu_p, T, cp, r, s, dev_status=status) for r in range(cp)]
            for r in range(cp):
                q_loc[r][:S] = q_full[parts[r].long()]
                do_loc[r][:S] = do_full[parts[r].long()]
                flops[s] += 14.0 * D * Hq * useful_pairs(parts[r].cpu().numpy().astype(np.int64), wl.cu_padded,
                                                          wl.cu_actual)
            if s == 0:
                order = torch.cat(parts).long()
                kg[:T], vg[:T] = k_phys[:T][order], v_phys[:T][order]
                k_in, v_in = k_buf, v_buf
            else:
                k_in, v_in = k_phys, v_phys

            def shares():
                for r in range(cp):
                    cpthd.partition_indices(cu_p, T, cp, r, s, out=idx_out, dev_status=status)
                    if s == 0:
                        cpthd.reorder_kv(kg, vg, cu_p, T, cp, 0, k_out=k_buf, v_out=v_buf, dev_status=status)
                    plan.build(cu_a, cu_p, T, r, s, status)
                    cpthd.attn_fwd(q_loc[r], k_in, v_in, plan, scale, o, lse, status)
                    cpthd.attn_bwd(q_loc[r], k_in, v_in, o, do_loc[r], lse, plan, scale, dq, dk, dv, status)

            shares()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                shares()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            total_ms += ms
            ms_by_strategy[s] += ms
    cpthd.check_dev_status(status)
    all_flops = flops[0] + flops[1]
    return {"microbatches": len(layouts), "shares": 2 * cp * len(layouts),
            "active_T": [int(min(wl.T for wl in layouts)), int(max(wl.T for wl in layouts))],
            "capacity_tokens": cap, "ms_per_sweep": total_ms,
            "tflops": all_flops / (total_ms * 1e-3) / 1e12,
            "tflops_by_strategy": {STRAT_NAME[s]: flops[s] / (ms_by_strategy[s] * 1e-3) / 1e12 for s in (0, 1)},
            "note": "every (micro-batch, strategy, rank) share's full step; useful fwd+bwd flops over GPU time"}


def long_context_shares(cpthd, torch, dev, status, reps=3):
    """The 70B-shaped long-context workload (T = 131,072 packed tokens, documents of 1 to 16,384 tokens, 64 q /
    8 kv heads, head dim 128, cp_size 8, contiguous strategy): ranks 0 and 7, each share's full step (partition,
    plan, forward, backward; contiguous ownership needs no restoration), timed between two events over reps
    repetitions after one untimed pass.  Tensor values are drawn on the GPU (timing only)."""
    wl = W.t131072_gqa64x8()
    T, cp, Hq, Hkv, D = wl.T, wl.cp, wl.Hq, wl.Hkv, wl.D
    S = T // cp
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)

    def randn(shape, sd):
        return (torch.randn(shape, generator=gen, device=dev) * sd).to(torch.bfloat16)

    k, v = randn((T, Hkv, D), 0.5), randn((T, Hkv, D), 0.5)
    cu_a = torch.from_numpy(wl.cu_actual).to(dev)
    cu_p = torch.from_numpy(wl.cu_padded).to(dev)
    plan = cpthd.AttnPlan(T, cp, Hq, Hkv, D, max_docs=wl.num_docs)
    idx = torch.empty(S, dtype=torch.int32, device=dev)
    o = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    dq = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    dk = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
    dv = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    out = []
    for r in (0, cp - 1):
        q, do = randn((S, Hq, D), 0.5), randn((S, Hq, D), 1.0)
        pairs = useful_pairs(cpthd.partition_indices(cu_p, T, cp, r, 1, dev_status=status).cpu().numpy()
                             .astype(np.int64), wl.cu_padded, wl.cu_actual)

        def share():
            cpthd.partition_indices(cu_p, T, cp, r, 1, out=idx, dev_status=status)
            plan.build(cu_a, cu_p, T, r, 1, status)
            cpthd.attn_fwd(q, k, v, plan, scale, o, lse, status)
            cpthd.attn_bwd(q, k, v, o, do, lse, plan, scale, dq, dk, dv, status)

        share()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            share()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out.append({"rank": r, "causal_pairs_per_head": int(pairs), "ms": ms,
                    "tflops": 14.0 * D * Hq * pairs / (ms * 1e-3) / 1e12})
        del q, do
    cpthd.check_dev_status(status)
    return {"T": T, "cp_size": cp, "num_q_heads": Hq, "num_kv_heads": Hkv, "num_docs": wl.num_docs,
            "strategy": "contiguous", "shares": out}


def short_mha_forward(cpthd, torch, dev, status, reps=10):
    """The forward-only workload of T = 8,192 packed tokens (documents of 256 to 2,048 tokens, 16 q / 16 kv
    heads, head dim 128, cp_size 2): ranks 0 and 1 under both strategies, each share's partition, restoration
    (DualChunkSwap), plan and forward, timed between two events over reps repetitions after one untimed pass.
    Tensor values are drawn on the GPU (timing only)."""
    wl = W.t8192_mha16()
    T, cp, Hq, Hkv, D = wl.T, wl.cp, wl.Hq, wl.Hkv, wl.D
    S = T // cp
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)

    def randn(shape, sd):
        return (torch.randn(shape, generator=gen, device=dev) * sd).to(torch.bfloat16)

    k_phys, v_phys = randn((T, Hkv, D), 0.5), randn((T, Hkv, D), 0.5)
    cu_a = torch.from_numpy(wl.cu_actual).to(dev)
    cu_p = torch.from_numpy(wl.cu_padded).to(dev)
    plan = cpthd.AttnPlan(T, cp, Hq, Hkv, D, max_docs=wl.num_docs)
    idx = torch.empty(S, dtype=torch.int32, device=dev)
    o = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    k_buf, v_buf = torch.empty_like(k_phys), torch.empty_like(v_phys)
    scale = 1.0 / math.sqrt(D)
    out, flops_all, ms_all = [], 0.0, 0.0
    for s in (0, 1):
        parts = [cpthd.partition_indices(cu_p, T, cp, r, s, dev_status=status) for r in range(cp)]
        order = torch.cat(parts).long()
        kg, vg = (k_phys[order].contiguous(), v_phys[order].contiguous()) if s == 0 else (k_phys, v_phys)
        k_in, v_in = (k_buf, v_buf) if s == 0 else (k_phys, v_phys)
        for r in range(cp):
            q = randn((S, Hq, D), 0.5)
            pairs = useful_pairs(parts[r].cpu().numpy().astype(np.int64), wl.cu_padded, wl.cu_actual)

            def share():
                cpthd.partition_indices(cu_p, T, cp, r, s, out=idx, dev_status=status)
                if s == 0:
                    cpthd.reorder_kv(kg, vg, cu_p, T, cp, 0, k_out=k_buf, v_out=v_buf, dev_status=status)
                plan.build(cu_a, cu_p, T, r, s, status)
                cpthd.attn_fwd(q, k_in, v_in, plan, scale, o, lse, status)

            share()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                share()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            fl = 4.0 * D * Hq * pairs
            flops_all += fl
            ms_all += ms
            out.append({"strategy": STRAT_NAME[s], "rank": r, "causal_pairs_per_head": int(pairs), "us": ms * 1e3,
                        "tflops": fl / (ms * 1e-3) / 1e12})
    cpthd.check_dev_status(status)
    return {"T": T, "cp_size": cp, "num_q_heads": Hq, "num_kv_heads": Hkv, "num_docs": wl.num_docs,
            "pass": "forward", "tflops": flops_all / (ms_all * 1e-3) / 1e12, "shares": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-allgathered", action="store_true",
                    help="skip the extra timing legs: the rank-major gathered K/V path and the HIP-graph replay of "
                         "the step (profiling runs: only the main step's launches)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after the timed region, run one plain copy of the K/V buffers (known bytes) through the "
                         "restoration kernel in contiguous mode, as the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's rank share only; run it with --gpus 1 (the library holds the per-rank "
              "kernels; the multi-GPU all-gather and reduce-scatter around them are not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import context_causal_thd_amd as cpthd

    dev = "cuda"
    wl = W.t32768_gqa32x8()
    T, cp, Hq, Hkv, D = wl.T, wl.cp, wl.Hq, wl.Hkv, wl.D
    S = T // cp
    log(f"workload: T={T} docs={wl.num_docs} Hq={Hq} Hkv={Hkv} D={D} cp={cp}")

    def bf16(x):
        return torch.from_numpy(W.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q_full, k_phys, v_phys, do_full = bf16(wl.q()), bf16(wl.k()), bf16(wl.v()), bf16(wl.do())
    cu_a = torch.from_numpy(wl.cu_actual).to(dev)
    cu_p = torch.from_numpy(wl.cu_padded).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    # per-share resident buffers (untimed set-up)
    shares = []
    for s, r in SHARES:
        idx = cpthd.partition_indices(cu_p, T, cp, r, s, dev_status=status)
        idx_l = idx.long()
        sh = dict(s=s, r=r, idx=torch.empty_like(idx), q=q_full[idx_l].contiguous(), do=do_full[idx_l].contiguous())
        if s == 0:   # simulated all-gather: rank-major concatenation of every rank's K/V rows
            parts = [cpthd.partition_indices(cu_p, T, cp, rr, s, dev_status=status).long() for rr in range(cp)]
            order = torch.cat(parts)
            sh["kg"], sh["vg"] = k_phys[order].contiguous(), v_phys[order].contiguous()
            sh["k"], sh["v"] = torch.empty_like(k_phys), torch.empty_like(v_phys)
        else:        # rank-major contiguous ownership: the gathered buffer is already physical order
            sh["kg"], sh["vg"] = k_phys, v_phys
            sh["k"], sh["v"] = k_phys, v_phys
        sh["plan"] = cpthd.AttnPlan(T, cp, Hq, Hkv, D, max_docs=wl.num_docs)
        sh["o"] = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
        sh["lse"] = torch.empty((S, Hq), dtype=torch.float32, device=dev)
        sh["dq"] = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
        sh["dk"] = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
        sh["dv"] = torch.empty((T, Hkv, D), dtype=torch.float32, device=dev)
        sh["pairs"] = useful_pairs(idx.cpu().numpy().astype(np.int64), wl.cu_padded, wl.cu_actual)
        shares.append(sh)
    del q_full, do_full
    torch.cuda.synchronize()
    cpthd.check_dev_status(status)

    row_bytes = Hkv * D * 2
    n_kernels = 6   # partition, reorder, plan, fwd, bwd-dq, bwd-dkdv

    def make_events():
        return ([[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)] for _ in shares],
                [[cpthd.HipEvents(2), cpthd.HipEvents(4)] for _ in shares])

    def step(evs):
        for i, sh in enumerate(shares):
            e, he = (evs[0][i], evs[1][i]) if evs else (None, None)
            if e:
                e[0][0].record()
            cpthd.partition_indices(cu_p, T, cp, sh["r"], sh["s"], out=sh["idx"], dev_status=status)
            if e:
                e[0][1].record()
                e[1][0].record()
            if sh["s"] == 0:
                cpthd.reorder_kv(sh["kg"], sh["vg"], cu_p, T, cp, 0, k_out=sh["k"], v_out=sh["v"],
                                 dev_status=status)
            if e:
                e[1][1].record()
                e[2][0].record()
            sh["plan"].build(cu_a, cu_p, T, sh["r"], sh["s"], status)
            if e:
                e[2][1].record()
            cpthd.attn_fwd(sh["q"], sh["k"], sh["v"], sh["plan"], wl.softmax_scale, sh["o"], sh["lse"], status,
                           events=he[0] if he else None)
            cpthd.attn_bwd(sh["q"], sh["k"], sh["v"], sh["o"], sh["do"], sh["lse"], sh["plan"], wl.softmax_scale,
                           sh["dq"], sh["dk"], sh["dv"], status, events=he[1] if he else None)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    cpthd.check_dev_status(status)
    log(f"warmup done ({args.warmup} steps)")

    # the timed steps: plain launches, nothing recorded between them
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(None)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    cpthd.check_dev_status(status)
    log(f"timed {args.steps} steps in {elapsed:.3f} s")

    # per-kernel durations: as many steps again, with events recorded around every launch
    events = [make_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k_step in range(args.steps):
        step(events[k_step])
    torch.cuda.synchronize()
    cpthd.check_dev_status(status)
    acc = np.zeros((len(shares), n_kernels))
    for evs, hevs in events:
        for i in range(len(shares)):
            for j in range(3):
                acc[i, j] += evs[i][j][0].elapsed_time(evs[i][j][1])
            acc[i, 3] += hevs[i][0].elapsed_ms(0, 1)
            acc[i, 4] += hevs[i][1].elapsed_ms(0, 1)
            acc[i, 5] += hevs[i][1].elapsed_ms(2, 3)

    # the same shares with attention reading the rank-major gathered K/V directly (no restoration pass)
    def step_allgathered(he):
        for i, sh in enumerate(shares):
            cpthd.partition_indices(cu_p, T, cp, sh["r"], sh["s"], out=sh["idx"], dev_status=status)
            sh["plan"].build(cu_a, cu_p, T, sh["r"], sh["s"], status)
            cpthd.attn_fwd(sh["q"], sh["kg"], sh["vg"], sh["plan"], wl.softmax_scale, sh["o"], sh["lse"], status,
                           events=he[i][0] if he else None, kv_allgathered=True)
            cpthd.attn_bwd(sh["q"], sh["kg"], sh["vg"], sh["o"], sh["do"], sh["lse"], sh["plan"], wl.softmax_scale,
                           sh["dq"], sh["dk"], sh["dv"], status, events=he[i][1] if he else None,
                           kv_allgathered=True)

    ag = None
    if not args.no_allgathered:
        for _ in range(args.warmup):
            step_allgathered(None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step_allgathered(None)
        torch.cuda.synchronize()
        ag_elapsed = time.perf_counter() - t0
        cpthd.check_dev_status(status)
        ag_events = [[[cpthd.HipEvents(2), cpthd.HipEvents(4)] for _ in shares] for _ in range(args.steps)]
        for k_step in range(args.steps):   # per-kernel durations: a second pass with events
            step_allgathered(ag_events[k_step])
        torch.cuda.synchronize()
        cpthd.check_dev_status(status)
        ag_acc = np.zeros((len(shares), 3))
        for he in ag_events:
            for i in range(len(shares)):
                ag_acc[i, 0] += he[i][0].elapsed_ms(0, 1)
                ag_acc[i, 1] += he[i][1].elapsed_ms(0, 1)
                ag_acc[i, 2] += he[i][1].elapsed_ms(2, 3)
        ag_acc /= args.steps
        log(f"allgathered path: {args.steps} steps in {ag_elapsed:.3f} s")
        ag = {"ms_per_step": ag_elapsed * 1e3 / args.steps}

    # the same step captured once in a HIP graph and replayed: the launch overhead a training loop that
    # captures its step would not pay (the kernels and their work are unchanged)
    graph_ms = None
    if not args.no_allgathered:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(None)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        cpthd.check_dev_status(status)
        del g
        log(f"graph replay: {args.steps} steps, {graph_ms:.3f} ms each")

    # the partition kernel alone at the million-token layout (T = 1,048,576 in 10,000 documents, cp_size 4),
    # every rank under both strategies: 20 calls captured in a HIP graph per (strategy, rank) and replayed, so
    # the host's launch rate does not enter the time
    part_big = None
    if not args.no_allgathered:
        cu_big_np, _ = W.t1m_10k_docs()
        T_big, cp_big = int(cu_big_np[-1]), 4
        cu_big = torch.from_numpy(cu_big_np).to(dev)
        idx_big = torch.empty(T_big // cp_big, dtype=torch.int32, device=dev)
        us = []
        for s_b in (0, 1):
            for r_b in range(cp_big):
                cpthd.partition_indices(cu_big, T_big, cp_big, r_b, s_b, out=idx_big, dev_status=status)
                torch.cuda.synchronize()
                g_b = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_b):
                    for _ in range(20):
                        cpthd.partition_indices(cu_big, T_big, cp_big, r_b, s_b, out=idx_big, dev_status=status)
                g_b.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(5):
                    g_b.replay()
                e1.record()
                torch.cuda.synchronize()
                us.append(e0.elapsed_time(e1) * 1e3 / 100)
                del g_b
        cpthd.check_dev_status(status)
        out_bytes = 4.0 * (T_big // cp_big)
        part_big = {"T": T_big, "num_docs": int(len(cu_big_np) - 1), "cp_size": cp_big,
                    "us_per_call_mean": float(np.mean(us)), "us_per_call_max": float(np.max(us)),
                    "out_bytes_per_call": out_bytes, "gbs": float(out_bytes / (np.mean(us) * 1e-6) / 1e9),
                    "note": "HIP-graph replay of 20 calls per (strategy, rank); 1 MiB of indices per call is "
                            "latency-bound"}
        log(f"partition at T={T_big}: {np.mean(us):.2f} us per call")

    dyn = None
    if not args.no_allgathered:
        dyn = dynamic_t_sweep(cpthd, torch, dev, status)
        log(f"dynamic-T sweep: {dyn['tflops']:.1f} TFLOP/s over {dyn['shares']} shares")
    shortf = None
    if not args.no_allgathered:
        shortf = short_mha_forward(cpthd, torch, dev, status)
        log(f"short MHA forward: {shortf['tflops']:.1f} TFLOP/s over {len(shortf['shares'])} shares")
    longc = None
    if not args.no_allgathered:
        longc = long_context_shares(cpthd, torch, dev, status)
        log("long context: " + ", ".join(f"rank {x['rank']} {x['tflops']:.1f} TFLOP/s" for x in longc["shares"]))

    # HBM ceiling for the restoration: a plain device-to-device copy of the same bytes (K and V), and the
    # restoration alone, each cold (a 512 MiB write before every rep evicts the 256 MiB last-level cache) and
    # the copy also warm (the source left in that cache, as inside the step)
    copy_src = torch.cat([k_phys.reshape(-1), v_phys.reshape(-1)])
    copy_dst = torch.empty_like(copy_src)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    sh0 = next(sh for sh in shares if sh["s"] == 0)

    def median_ms(fn, cold):
        ms = []
        for rep in range(7):
            if cold:
                flush.fill_(rep)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if rep:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    moved = 2.0 * 2.0 * T * Hkv * D * 2     # K and V, read + write
    copy_cold = moved / (median_ms(lambda: copy_dst.copy_(copy_src), True) * 1e-3) / 1e9
    copy_warm = moved / (median_ms(lambda: copy_dst.copy_(copy_src), False) * 1e-3) / 1e9
    reorder_cold = moved / (median_ms(lambda: cpthd.reorder_kv(sh0["kg"], sh0["vg"], cu_p, T, cp, 0, k_out=sh0["k"],
                                                              v_out=sh0["v"], dev_status=status), True) * 1e-3) / 1e9
    cpthd.check_dev_status(status)
    del flush, copy_dst, copy_src

    if args.calibration_copy:
        k2, v2 = torch.empty_like(k_phys), torch.empty_like(v_phys)
        cpthd.reorder_kv(k_phys, v_phys, cu_p, T, cp, 1, k_out=k2, v_out=v2, dev_status=status)
        torch.cuda.synchronize()
        log(f"calibration copy: {2 * k_phys.numel() * 2} bytes read and written")

    # pure-GPU step time: the per-kernel event durations of one step
    per_kernel_ms = acc / args.steps
    gpu_step_ms = float(per_kernel_ms.sum())
    wall_step_ms = elapsed * 1e3 / args.steps
    pairs = np.array([sh["pairs"] for sh in shares], dtype=np.float64)
    flops_fwd = 4.0 * D * Hq * pairs
    flops_bwd = 10.0 * D * Hq * pairs
    step_flops = float(np.sum(flops_fwd + flops_bwd))
    value = step_flops / (wall_step_ms * 1e-3) / 1e12

    names = ["partition", "reorder", "plan", "attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv"]
    kernel_ms = {n: float(per_kernel_ms[:, j].sum()) for j, n in enumerate(names)}
    # algorithmic flops per kernel: fwd = 4DHqN; of the backward's 10DHqN, the key-tile pass computes the
    # score and dP recompute plus dK and dV (8DHqN), the query-tile pass dQ (2DHqN; its recompute is extra)
    algo = {"attn_fwd": flops_fwd, "attn_bwd_dkdv": 0.8 * flops_bwd, "attn_bwd_dq": 0.2 * flops_bwd}
    dominant = max(algo, key=lambda n: kernel_ms[n])
    j = names.index(dominant)
    achieved = float(np.sum(algo[dominant]) / (kernel_ms[dominant] * 1e-3) / 1e12)
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dominant),
                "traffic_unit": "bytes per launch (HBM, calibrated FETCH_SIZE + WRITE_SIZE)",
                "avg_launch_us": float(per_kernel_ms[:, j].mean() * 1e3)}

    dcs = [i for i, sh in enumerate(shares) if sh["s"] == 0]
    part_bytes = 4.0 * S
    reorder_bytes = 2.0 * 2.0 * T * row_bytes      # read + write of K and V
    breakdown = {
        "per_share": [
            {"strategy": STRAT_NAME[sh["s"]], "rank": sh["r"], "causal_pairs_per_head": int(sh["pairs"]),
             "fwd_tflops": float(flops_fwd[i] / (per_kernel_ms[i, 3] * 1e-3) / 1e12),
             "bwd_tflops": float(flops_bwd[i] / ((per_kernel_ms[i, 4] + per_kernel_ms[i, 5]) * 1e-3) / 1e12),
             "fwd_bwd_tflops": float((flops_fwd[i] + flops_bwd[i]) / (per_kernel_ms[i, 3:].sum() * 1e-3) / 1e12),
             "ms": {n: float(per_kernel_ms[i, jj]) for jj, n in enumerate(names)}}
            for i, sh in enumerate(shares)],
        "kernel_ms_per_step": kernel_ms,
        "attn_fwd_bwd_tflops": float(step_flops / (per_kernel_ms[:, 3:].sum() * 1e-3) / 1e12),
        "attn_frac_of_bf16_peak": float(step_flops / (per_kernel_ms[:, 3:].sum() * 1e-3) / 1e12 / PEAK_BF16_TFLOPS),
        "partition_gbs": float(part_bytes / (per_kernel_ms[:, 0].mean() * 1e-3) / 1e9),
        "partition_million_tokens": part_big,
        # the dynamic-T micro-batch sweep on capacity buffers (65,536 tokens): every share of 16 micro-batches
        "dynamic_t_sweep": dyn,
        # the 70B-shaped long-context workload (T = 131,072, 64 q / 8 kv heads, cp_size 8): contiguous ranks 0, 7
        "long_context_shares": longc,
        # the forward-only T = 8,192 workload (16 q / 16 kv heads, cp_size 2): both strategies, ranks 0 and 1
        "short_mha_forward": shortf,
        "reorder_gbs": float(reorder_bytes / (per_kernel_ms[dcs, 1].mean() * 1e-3) / 1e9),
        "reorder_frac_of_hbm_peak": float(reorder_bytes / (per_kernel_ms[dcs, 1].mean() * 1e-3) / 1e9 / PEAK_HBM_GBS),
        "reorder_gbs_cold": reorder_cold,
        "device_copy_gbs_same_bytes": {"cold": copy_cold, "warm": copy_warm},
        "gpu_kernel_ms_per_step": gpu_step_ms,
        "shader_clock_during_timed_steps": clock.summary(),
        # attention reading the all-gathered (rank-major) K/V through the inverse partition map: partition +
        # plan + fwd + bwd per share, no restoration pass; dK/dV come out in the gathered order
        "allgathered_path": None if ag is None else {
            "ms_per_step": ag["ms_per_step"],
            "tflops": step_flops / (ag["ms_per_step"] * 1e-3) / 1e12,
            "kernel_ms_per_step": {n: float(ag_acc[:, jj].sum())
                                   for jj, n in enumerate(["attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv"])},
        },
        # the main step (restoration path) replayed from a HIP graph, same kernels and inputs
        "graph_replayed_step": None if graph_ms is None else {
            "ms_per_step": graph_ms, "tflops": step_flops / (graph_ms * 1e-3) / 1e12},
    }

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, args.cpu_budget)

    out = {
        "metric": "useful causal attn TFLOP/s per CP-rank share (fwd+bwd) + % bf16 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "t32768_gqa32x8: T=32768 packed bf16 tokens, 32 q / 8 kv heads, head_dim 128, log-normal "
                               "doc lengths (median 1024, sigma 1) clipped to [64,8192] padded to x8, cp_size=4; "
                               "shares dcs r0, dcs r3, contiguous r0, contiguous r3; partition + reorder + plan + "
                               "attention fwd + bwd per share",
                   "T": T, "cp_size": cp, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "num_docs": wl.num_docs, "parallelism": "one CP rank share per call, 1 GPU"},
        "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
