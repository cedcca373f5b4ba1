#!/usr/bin/env python3
"""Benchmark of the paged KV-cache hot path on one MI355X.

Metric: paged decode KV-read GB/s (fraction of the 8 TB/s HBM peak) and
microseconds per decode step; prefill TFLOP/s.

One step = one pass of the decode hot path over the LLaMA-7B-shaped batch
(8 sequences x 2048 tokens, 32/32 heads, head_dim 128, block_size 16, pool
4096 blocks, fp16): the new token of every sequence is scattered into the
pool through slot_mapping (paged_kv_write), then every sequence's query
attends over its 2048 paged tokens (paged_attention_decode; on this batch
one workgroup per whole context, no split and no reduce). Inputs are
synthetic (N(0,1) values,
a seeded random block permutation) and resident in HBM before timing. A
1 GiB buffer is read between timed steps so that the 256 MB Infinity Cache
does not serve the KV reads (a read, so that no dirty lines are left behind).

Prints ONE JSON line. Extra fields carry the packed-prefill TFLOP/s, the
ragged GQA and long-context decode figures, the roofline of the dominant
kernel and the CPU oracle baseline.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_fp16_traffic.json")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix peak, TFLOP/s
FLUSH_BYTES = 1 << 30          # read between timed steps (4x the Infinity Cache)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the decode step workload")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the packed causal prefill workload (for counter runs)")
    ap.add_argument("--prefill-workload", type=int, default=4, choices=(4, 6),
                    help="with --prefill-only: the packed prefill (4) or the mixed batch (6)")
    return ap.parse_args()


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter
    passes (FETCH_SIZE / WRITE_SIZE, scaled by the factors measured on a
    plain 1 GiB read and a plain 1 GiB fill). None when the kernel sources
    have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if source_digest(rec["sources"]) != rec["sources_sha256"]:
        return None, rec
    kib = rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] + \
        rec["write_kib_per_dispatch"] * rec["write_scale"]
    return int(round(kib * 1024)), rec


class Timer:
    """Per-step HIP events on the stream the library launches on."""

    def __init__(self, torch, n):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]


class KernelEvents:
    """hipEvent_t pairs (timing enabled) that the library's measurement hook
    (pkv_time_next_kernel) has one kernel launch record at its own dispatch
    start and end: the kernel's execution time, as a kernel trace reports
    it, without the event-packet gaps that events around a call include.
    The events come from the HIP runtime this process already loaded."""

    def __init__(self, n):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))

    def arm(self, binding, i):
        binding.time_next_kernel(*self.pairs[i])

    def ms(self, i):
        out = self.ct.c_float()
        a, b = self.pairs[i]
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a),
                                        self.ct.c_void_p(b)):
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(self.ct.c_void_p(a))
            self.hip.hipEventDestroy(self.ct.c_void_p(b))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the library has no "
                                   "multi-GPU path (use --gpus 1)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_39_amd import binding
    from paged_kv_cache_39_amd import workloads as wl

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    binding.lib()  # fail loudly before any timing if the library is missing

    flush = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, dtype=torch.float32,
                                                  device=dev)

    def evict():
        if flush is not None:
            flush.sum()

    def ramp_clocks(seconds=0.3):
        """Untimed: keep the GPU busy for a moment so that its shader clock
        has left the idle level before anything is timed (an idle part
        starts far below its peak clock and ramps up under load)."""
        busy = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                busy.sum()
            torch.cuda.synchronize()
        del busy

    def tdt(dtype):
        return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]

    def ints(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    if args.prefill_only:
        # the packed causal prefill alone: W warm-up calls, then K timed calls
        m = wl.workload(args.prefill_workload, values=False)
        dtp = tdt(m.dtype)
        k = torch.randn(m.pool_shape(), dtype=dtp, device=dev)
        v = torch.randn_like(k)
        q = torch.randn(int(m.cu_seqlens_q[-1]), m.num_q_heads, m.head_dim, dtype=dtp, device=dev)
        out = torch.empty_like(q)
        cu, bt, sl = ints(m.cu_seqlens_q), ints(m.block_table), ints(m.seq_lens)
        ramp_clocks()
        for _ in range(args.warmup):
            evict()
            binding.paged_attention_varlen(out, q, cu, k, v, bt, sl, True)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            evict()
            a.record()
            binding.paged_attention_varlen(out, q, cu, k, v, bt, sl, True)
            b.record()
        torch.cuda.synchronize()
        mu = statistics.mean([a.elapsed_time(b) for a, b in evs])
        # the kernel alone: dispatch-recorded events, one call each
        ke = KernelEvents(args.steps)
        for i in range(args.steps):
            evict()
            ke.arm(binding, i)
            binding.paged_attention_varlen(out, q, cu, k, v, bt, sl, True)
        torch.cuda.synchronize()
        kms = [ke.ms(i) for i in range(args.steps)]
        ke.close()
        km = statistics.mean(kms)
        fl = m.prefill_flops()
        print(json.dumps({"workload": m.name, "steps": args.steps, "us": round(mu * 1e3, 2),
                          "tflops": round(fl / (mu * 1e-3) / 1e12, 2), "flops": fl,
                          "kernel_us": round(km * 1e3, 2),
                          "kernel_us_min": round(min(kms) * 1e3, 2),
                          "kernel_tflops": round(fl / (km * 1e-3) / 1e12, 2)}))
        return

    def decode_setup(meta):
        dt = tdt(meta.dtype)
        shape = meta.pool_shape()
        k = torch.randn(shape, dtype=dt, device=dev)
        v = torch.randn(shape, dtype=dt, device=dev)
        q = torch.randn(meta.num_seqs, meta.num_q_heads, meta.head_dim, dtype=dt, device=dev)
        out = torch.empty_like(q)
        bt, ctx = ints(meta.block_table), ints(meta.seq_lens)
        ws_bytes = binding.paged_attention_decode_workspace_size(
            meta.num_seqs, meta.num_q_heads, meta.head_dim, meta.max_blocks_per_seq,
            meta.block_size)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        return dict(k=k, v=v, q=q, out=out, bt=bt, ctx=ctx, ws=ws)

    def run_decode(meta, t):
        binding.paged_attention_decode(t["out"], t["q"], t["k"], t["v"], t["bt"], t["ctx"],
                                       meta.block_size, meta.scale, workspace=t["ws"])

    # ------------------------------------------------------------------
    # the step workload: LLaMA-7B-shaped decode, new token written + attended
    # ------------------------------------------------------------------
    meta = wl.workload(2, values=False)
    t = decode_setup(meta)
    dt = tdt(meta.dtype)
    new_key = torch.randn(meta.num_seqs, meta.num_kv_heads, meta.head_dim, dtype=dt, device=dev)
    new_val = torch.randn_like(new_key)
    new_slots = ints(meta.slot_mapping[meta.new_token_rows])

    def step():
        """One decode step through the fused call: the new tokens are written
        and attended in one launch (paged_kv_write_decode)."""
        binding.paged_kv_write_decode(t["out"], t["q"], t["k"], t["v"], new_key, new_val,
                                      new_slots, t["bt"], t["ctx"], meta.block_size, meta.scale,
                                      workspace=t["ws"])

    def kernel_pass(fn, n):
        """ms of the first kernel of each of n calls, from events the kernel
        dispatch records (pkv_time_next_kernel)."""
        ke = KernelEvents(n)
        for i in range(n):
            evict()
            ke.arm(binding, i)
            fn()
        torch.cuda.synchronize()
        kms = [ke.ms(i) for i in range(n)]
        ke.close()
        return kms

    ramp_clocks()
    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    clocks0 = gpu_clocks()
    tm = Timer(torch, args.steps)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        e0, e1, _ = tm.ev[i]
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b, _ in tm.ev]
    # kernel-level pass right after the timed steps, same inputs and cache
    # flush: the fused kernel records dispatch events (arming them makes the
    # runtime add gaps around the call, so the timed steps run unarmed)
    kern_ms = kernel_pass(step, args.steps)
    kern_mean = statistics.mean(kern_ms)
    e = wl.ELEM_BYTES[meta.dtype]
    # the step reads every context token's K/V once (the new token's from
    # key/value), q, the live table entries, the lengths and the slots, and
    # writes out and the new rows
    new_rows_bytes = 2 * meta.num_seqs * meta.num_kv_heads * meta.head_dim * e
    step_bytes = meta.decode_bytes() + new_rows_bytes + 4 * meta.num_seqs
    kern_gbs = step_bytes / (kern_mean * 1e-3) / 1e9
    ms_per_step = statistics.mean(step_ms)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # for comparison: the same step as two calls (paged_kv_write, then
    # paged_attention_decode), and the decode call's own kernel; warmed up
    # first, like the fused step (a first call pays the kernels' loading)
    for _ in range(args.warmup):
        evict()
        binding.paged_kv_write(t["k"], t["v"], new_key, new_val, new_slots)
        run_decode(meta, t)
    torch.cuda.synchronize()
    tm2 = Timer(torch, args.steps)
    for i in range(args.steps):
        evict()
        e0, e1, e2 = tm2.ev[i]
        e0.record()
        binding.paged_kv_write(t["k"], t["v"], new_key, new_val, new_slots)
        e1.record()
        run_decode(meta, t)
        e2.record()
    torch.cuda.synchronize()
    two_ms = [a.elapsed_time(c) for a, b, c in tm2.ev]
    dec_ms = [b.elapsed_time(c) for a, b, c in tm2.ev]
    write_ms = [a.elapsed_time(b) for a, b, c in tm2.ev]
    dec_kern_ms = kernel_pass(lambda: run_decode(meta, t), args.steps)
    dec_mean = statistics.mean(dec_ms)
    dec_gbs = meta.decode_bytes() / (dec_mean * 1e-3) / 1e9

    result = {
        "metric": "paged decode KV-read GB/s (% of HBM peak) + us/step; prefill TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: N(0,1) fp16 K/V/q, seeded random block permutation, inputs resident in HBM",
        "config": {"workload": "llama7b-shaped paged decode step: write 1 new token/seq via "
                               "slot_mapping and decode, one fused call", "batch": meta.num_seqs,
                   "context": int(meta.seq_lens[0]), "q_heads": meta.num_q_heads,
                   "kv_heads": meta.num_kv_heads, "head_dim": meta.head_dim,
                   "block_size": meta.block_size, "pool_blocks": meta.num_blocks,
                   "partition_tokens": binding.decode_partition_tokens(
                       meta.num_seqs, meta.num_q_heads, meta.num_kv_heads,
                       meta.max_blocks_per_seq, meta.block_size, torch.float16),
                   "cache_flush_between_steps": flush is not None},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)) * 1e3, 2),
                                round(float(np.percentile(step_ms, 90)) * 1e3, 2)],
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "step_kernel_us": round(kern_mean * 1e3, 2),
        "step_kernel_us_median": round(statistics.median(kern_ms) * 1e3, 2),
        "step_kernel_us_p10_p90": [round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
                                   round(float(np.percentile(kern_ms, 90)) * 1e3, 2)],
        "two_call_us_per_step": round(statistics.mean(two_ms) * 1e3, 2),
        "kv_write_call_us": round(statistics.mean(write_ms) * 1e3, 2),
        "decode_call_us": round(dec_mean * 1e3, 2),
        "decode_call_gbs": round(dec_gbs, 1),
        "decode_kernel_us": round(statistics.mean(dec_kern_ms) * 1e3, 2),
        "decode_kernel_gbs": round(meta.decode_bytes() / statistics.mean(dec_kern_ms) / 1e6, 1),
        "step_bytes": step_bytes,
        "timed_wall_s": round(wall, 4),
    }
    traffic, trec = measured_traffic()
    result["roofline"] = {
        "kernel": "decode_mfma_kernel, fused-write instance (the one launch of a "
                  "paged_kv_write_decode call on this batch: 8-wave workgroups, one whole "
                  "2048-token context each, no split)",
        "bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
        "algorithmic_bytes_per_launch": step_bytes,
        "timing": "per launch: HIP events recorded by the kernel dispatch itself "
                  "(hipExtLaunchKernel through pkv_time_next_kernel) on the launch stream, "
                  "mean over a pass of as many calls as timed steps that follows them "
                  "(same inputs, same cache flush); events around the whole call "
                  "(us_per_step) add the event-packet gaps",
    }
    if trec is not None:
        result["roofline"]["traffic_source"] = os.path.relpath(TRAFFIC_FILE, ROOT)
    del t, new_key, new_val
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------
    # other paths of the hot loop (same method: events per call, cache flush)
    # ------------------------------------------------------------------
    def time_calls(fn, n, warm=3):
        """Per call: ms between events around the call; then, in a pass of
        its own, ms of the call's first kernel from dispatch-recorded events."""
        for _ in range(warm):
            evict()
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            evict()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs], kernel_pass(fn, n)

    if not args.no_extra:
        n_extra = max(5, min(args.steps, 20))
        extra = {}
        for c in (3, 5):
            m = wl.workload(c, values=False)
            tt = decode_setup(m)
            ms, kms = time_calls(lambda: run_decode(m, tt), n_extra)
            mu = statistics.mean(ms)
            gbs = m.decode_bytes() / (mu * 1e-3) / 1e9
            extra[m.name] = {"us": round(mu * 1e3, 2), "gbs": round(gbs, 1),
                             "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "bytes": m.decode_bytes(),
                             "kernel_us": round(statistics.mean(kms) * 1e3, 2),
                             "partition_tokens": binding.decode_partition_tokens(
                                 m.num_seqs, m.num_q_heads, m.num_kv_heads,
                                 m.max_blocks_per_seq, m.block_size, tdt(m.dtype))}
            if c == 5:
                # the same call with the workload's stated 512-token
                # partitions (4-wave workgroups + the reduce) instead of the
                # launch plan's
                binding.decode_partition_override(512)
                try:
                    ms5, kms5 = time_calls(lambda: run_decode(m, tt), n_extra)
                finally:
                    binding.decode_partition_override(0)
                mu5 = statistics.mean(ms5)
                extra[m.name]["partition_512"] = {
                    "us": round(mu5 * 1e3, 2),
                    "gbs": round(m.decode_bytes() / (mu5 * 1e-3) / 1e9, 1),
                    "hbm_peak_frac": round(m.decode_bytes() / (mu5 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                           4),
                    "kernel_us": round(statistics.mean(kms5) * 1e3, 2),
                    "partition_tokens": 512}
            if c == 3:
                # the ragged batch's decode step too (write + attention): one
                # fused call, and the two calls
                nk = torch.randn(m.num_seqs, m.num_kv_heads, m.head_dim, dtype=tdt(m.dtype),
                                 device=dev)
                nv = torch.randn_like(nk)
                ns = ints(m.slot_mapping[m.new_token_rows])
                ms, _ = time_calls(lambda: binding.paged_kv_write_decode(
                    tt["out"], tt["q"], tt["k"], tt["v"], nk, nv, ns, tt["bt"], tt["ctx"],
                    m.block_size, m.scale, workspace=tt["ws"]), n_extra)

                def two_calls():
                    binding.paged_kv_write(tt["k"], tt["v"], nk, nv, ns)
                    run_decode(m, tt)
                ms2, _ = time_calls(two_calls, n_extra)
                extra[m.name]["step_us"] = round(statistics.mean(ms) * 1e3, 2)
                extra[m.name]["two_call_step_us"] = round(statistics.mean(ms2) * 1e3, 2)
                del nk, nv
            del tt
            torch.cuda.empty_cache()
        # int8 cache on the LLaMA-7B shape: the same decode over 1-byte codes
        # (per-kv-head scales), fp16 q/out; algorithmic bytes count the codes
        m = wl.workload(2, values=False)
        ks, vs = wl.int8_scales(m.num_kv_heads)
        k8 = torch.randint(-127, 128, m.pool_shape(), dtype=torch.int8, device=dev)
        v8 = torch.randint_like(k8, -127, 128)
        q8 = torch.randn(m.num_seqs, m.num_q_heads, m.head_dim, dtype=tdt(m.dtype), device=dev)
        o8 = torch.empty_like(q8)
        ksd, vsd = torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev)
        bt8, ctx8 = ints(m.block_table), ints(m.seq_lens)
        ws8 = torch.empty(max(1, binding.paged_attention_decode_workspace_size(
            m.num_seqs, m.num_q_heads, m.head_dim, m.max_blocks_per_seq, m.block_size)),
            dtype=torch.uint8, device=dev)
        ms, kms = time_calls(lambda: binding.paged_attention_decode_int8(
            o8, q8, k8, v8, ksd, vsd, bt8, ctx8, m.block_size, m.scale, workspace=ws8), n_extra)
        mu = statistics.mean(ms)
        b8 = m.decode_bytes() - m.kv_bytes_read() // 2
        gbs = b8 / (mu * 1e-3) / 1e9
        # its decode step (write the 8 new rows as codes + attend): one fused
        # call, and the two calls
        nk8 = torch.randn(m.num_seqs, m.num_kv_heads, m.head_dim, dtype=tdt(m.dtype), device=dev)
        nv8 = torch.randn_like(nk8)
        ns8 = ints(m.slot_mapping[m.new_token_rows])
        ms_f, kms_f = time_calls(lambda: binding.paged_kv_write_decode_int8(
            o8, q8, k8, v8, nk8, nv8, ksd, vsd, ns8, bt8, ctx8, m.block_size, m.scale,
            workspace=ws8), n_extra)

        def two_calls8():
            binding.paged_kv_write_int8(k8, v8, nk8, nv8, ksd, vsd, ns8)
            binding.paged_attention_decode_int8(o8, q8, k8, v8, ksd, vsd, bt8, ctx8,
                                                m.block_size, m.scale, workspace=ws8)
        ms_2, _ = time_calls(two_calls8, n_extra)
        extra["int8_kv_decode_llama7b_b8_ctx2048"] = {
            "us": round(mu * 1e3, 2), "gbs": round(gbs, 1),
            "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": b8,
            "kernel_us": round(statistics.mean(kms) * 1e3, 2),
            "step_us": round(statistics.mean(ms_f) * 1e3, 2),
            "step_kernel_us": round(statistics.mean(kms_f) * 1e3, 2),
            "two_call_step_us": round(statistics.mean(ms_2) * 1e3, 2)}
        del nk8, nv8
        del k8, v8
        torch.cuda.empty_cache()
        for c in (4, 6):
            # 4: packed causal prefill; 6: decode + multi-token decode + chunked
            # prefill rows in one packed call (its KV GB/s is reported as well)
            m = wl.workload(c, values=False)
            dtp = tdt(m.dtype)
            k = torch.randn(m.pool_shape(), dtype=dtp, device=dev)
            v = torch.randn_like(k)
            q = torch.randn(int(m.cu_seqlens_q[-1]), m.num_q_heads, m.head_dim, dtype=dtp,
                            device=dev)
            out = torch.empty_like(q)
            cu, bt, sl = ints(m.cu_seqlens_q), ints(m.block_table), ints(m.seq_lens)
            ms, kms = time_calls(lambda: binding.paged_attention_varlen(out, q, cu, k, v, bt, sl, True),
                            n_extra)
            mu = statistics.mean(ms)
            fl = m.prefill_flops()
            extra[m.name] = {"us": round(mu * 1e3, 2),
                             "tflops": round(fl / (mu * 1e-3) / 1e12, 2),
                             "bf16_peak_frac": round(fl / (mu * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                             "flops": fl, "total_q": int(m.cu_seqlens_q[-1]),
                             "kernel_us": round(statistics.mean(kms) * 1e3, 2),
                             "kernel_tflops": round(fl / (statistics.mean(kms) * 1e-3) / 1e12, 2)}
            if c == 6:
                extra[m.name]["kv_gbs"] = round(m.kv_bytes_read() / (mu * 1e-3) / 1e9, 1)
                extra[m.name]["kv_bytes"] = m.kv_bytes_read()
                # the same batch through the split call (workspace from the binding's cache)
                ms, _ = time_calls(lambda: binding.paged_attention_varlen_split(
                    out, q, cu, k, v, bt, sl, True), n_extra)
                mus = statistics.mean(ms)
                extra[m.name]["split_us"] = round(mus * 1e3, 2)
                extra[m.name]["split_kv_gbs"] = round(m.kv_bytes_read() / (mus * 1e-3) / 1e9, 1)
            if c == 4:
                result["prefill_tflops"] = extra[m.name]["tflops"]
            del k, v, q, out
            torch.cuda.empty_cache()
        # mixed batch over long contexts: 8 decode rows at 32768 tokens and two
        # 512-query chunks over 2048 keys (32/8 heads, D 128, bs 16, bf16),
        # plain call vs split call
        m = wl.varlen_case(1007, [1] * 8 + [512, 512], [32768] * 8 + [2048, 2048], 32, 8, 128,
                           16, "bf16", causal=True, values=False, name="mixed_long_decode_32k_bf16")
        dtp = tdt(m.dtype)
        k = torch.randn(m.pool_shape(), dtype=dtp, device=dev)
        v = torch.randn_like(k)
        q = torch.randn(int(m.cu_seqlens_q[-1]), m.num_q_heads, m.head_dim, dtype=dtp, device=dev)
        out = torch.empty_like(q)
        cu, bt, sl = ints(m.cu_seqlens_q), ints(m.block_table), ints(m.seq_lens)
        ms, _ = time_calls(lambda: binding.paged_attention_varlen(out, q, cu, k, v, bt, sl, True),
                           n_extra)
        msx, _ = time_calls(lambda: binding.paged_attention_varlen_split(
            out, q, cu, k, v, bt, sl, True), n_extra)
        mu, mus = statistics.mean(ms), statistics.mean(msx)
        extra[m.name] = {"us": round(mu * 1e3, 2), "split_us": round(mus * 1e3, 2),
                         "kv_gbs": round(m.kv_bytes_read() / (mu * 1e-3) / 1e9, 1),
                         "split_kv_gbs": round(m.kv_bytes_read() / (mus * 1e-3) / 1e9, 1),
                         "kv_bytes": m.kv_bytes_read(), "flops": m.prefill_flops()}
        del k, v, q, out
        torch.cuda.empty_cache()
        # variants: ALiBi + a sliding window. Decode on the LLaMA-7B shape
        # (window 1024: bytes = the visible keys' rows), packed prefill of
        # workload 4 (window 512: flops = allowed pairs)
        m = wl.workload(2, values=False)
        tt = decode_setup(m)
        slopes = torch.from_numpy(wl.alibi_slopes(m.num_q_heads)).to(dev)
        win = 1024
        ms, kms = time_calls(lambda: binding.paged_attention_decode_ex(
            tt["out"], tt["q"], tt["k"], tt["v"], tt["bt"], tt["ctx"], m.block_size, m.scale,
            slopes, win, workspace=tt["ws"]), n_extra)
        mu = statistics.mean(ms)
        vis = sum(min(int(n), win + 1) for n in m.seq_lens)
        eb = 2
        bw = vis * 2 * m.num_kv_heads * m.head_dim * eb + 2 * m.num_seqs * m.num_q_heads * m.head_dim * eb
        extra["decode_alibi_window1024_llama7b"] = {
            "us": round(mu * 1e3, 2), "gbs": round(bw / (mu * 1e-3) / 1e9, 1),
            "hbm_peak_frac": round(bw / (mu * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": bw,
            "kernel_us": round(statistics.mean(kms) * 1e3, 2)}
        del tt
        torch.cuda.empty_cache()
        m = wl.workload(4, values=False)
        dtp = tdt(m.dtype)
        k = torch.randn(m.pool_shape(), dtype=dtp, device=dev)
        v = torch.randn_like(k)
        q = torch.randn(int(m.cu_seqlens_q[-1]), m.num_q_heads, m.head_dim, dtype=dtp, device=dev)
        out = torch.empty_like(q)
        cu, bt, sl = ints(m.cu_seqlens_q), ints(m.block_table), ints(m.seq_lens)
        slopes = torch.from_numpy(wl.alibi_slopes(m.num_q_heads)).to(dev)
        win = 512
        ms, kms = time_calls(lambda: binding.paged_attention_varlen_ex(
            out, q, cu, k, v, bt, sl, True, slopes, win), n_extra)
        mu = statistics.mean(ms)
        pairs = 0
        for b in range(m.num_seqs):
            lq = int(m.cu_seqlens_q[b + 1] - m.cu_seqlens_q[b])
            pairs += sum(min(i, win) + 1 for i in range(lq))      # Lq == Lk here
        fl = 4 * m.head_dim * m.num_q_heads * pairs
        extra["prefill_alibi_window512_16seq"] = {
            "us": round(mu * 1e3, 2), "tflops": round(fl / (mu * 1e-3) / 1e12, 2),
            "bf16_peak_frac": round(fl / (mu * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4), "flops": fl,
            "kernel_us": round(statistics.mean(kms) * 1e3, 2)}
        del k, v, q, out
        torch.cuda.empty_cache()
        # block manager: host cost of one decode step's scheduling (256
        # sequences at 1024 tokens, bs 16: append one token each, build the
        # block table and lengths, take the copies), and the device block copy
        import numpy as np
        nseq, bsz = 256, 16
        bm = binding.BlockManager(nseq * (1024 // bsz + 8), bsz)
        for sq in range(nseq):
            bm.add_sequence(sq)
            bm.append(sq, 1024)
        slots = np.empty(nseq, np.int32)
        ids = np.arange(nseq, dtype=np.int64)
        n_host = 200
        t0 = time.perf_counter()
        for _ in range(n_host):
            bm.append_each(ids, 1, slots)
            bm.block_table(ids, 1024 // bsz + 8)
            bm.take_copies()
        host_us = (time.perf_counter() - t0) / n_host * 1e6
        bm.close()
        m = wl.workload(2, values=False)
        kc = torch.randn(m.pool_shape(), dtype=tdt(m.dtype), device=dev)
        vc = torch.randn_like(kc)
        npairs = 1024
        perm = torch.randperm(m.num_blocks)
        pairs = torch.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).to(torch.int32).to(dev)
        ms, kms = time_calls(lambda: binding.paged_kv_copy_blocks(kc, vc, pairs), n_extra)
        mu = statistics.mean(ms)
        cbytes = 2 * 2 * npairs * m.block_size * m.num_kv_heads * m.head_dim * 2 + npairs * 8
        extra["block_manager_decode_step_b256"] = {
            "host_us_per_step": round(host_us, 2),
            "note": "pkv_bm_append_each (1 token for each of 256 sequences) + block_table + "
                    "take_copies, one host thread, through the Python binding"}
        extra["copy_blocks_fp16_1024_blocks"] = {
            "us": round(mu * 1e3, 2), "gbs": round(cbytes / (mu * 1e-3) / 1e9, 1),
            "hbm_peak_frac": round(cbytes / (mu * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": cbytes}
        del kc, vc
        torch.cuda.empty_cache()
        # the packed prefill's KV write: every token of the 16 sequences
        # (slot_mapping over the bs-128 pool), 2 KiB rows of K and of V
        m = wl.workload(4, values=False)
        kc = torch.empty(m.pool_shape(), dtype=tdt(m.dtype), device=dev)
        vc = torch.empty_like(kc)
        ntok = int(m.slot_mapping.shape[0])
        nkey = torch.randn(ntok, m.num_kv_heads, m.head_dim, dtype=tdt(m.dtype), device=dev)
        nval = torch.randn_like(nkey)
        smap = ints(m.slot_mapping)
        ms, kms = time_calls(lambda: binding.paged_kv_write(kc, vc, nkey, nval, smap), n_extra)
        mu = statistics.mean(ms)
        wbytes = 2 * 2 * ntok * m.num_kv_heads * m.head_dim * wl.ELEM_BYTES[m.dtype] + 4 * ntok
        extra["kv_write_prefill_16seq_bf16"] = {
            "us": round(mu * 1e3, 2), "gbs": round(wbytes / (mu * 1e-3) / 1e9, 1),
            "hbm_peak_frac": round(wbytes / (mu * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes": wbytes, "tokens": ntok,
            "kernel_us": round(statistics.mean(kms) * 1e3, 2)}
        del kc, vc, nkey, nval
        torch.cuda.empty_cache()
        result["other_workloads"] = extra

    result["gpu_clocks"] = {"before": clocks0, "after": gpu_clocks()}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()

    print(json.dumps(result), flush=True)


def gpu_clocks():
    """Current shader and memory clock levels of the GPU (the DPM level the
    driver marks active in sysfs), or None where sysfs does not show them."""
    import glob
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(card, name)) as f:
                    cur = [ln.split(":", 1)[1].strip().rstrip("*").strip()
                           for ln in f if ln.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                out.setdefault(os.path.basename(os.path.dirname(card)), {})[name[3:]] = cur[0]
    return out or None


def cpu_baseline():
    """The oracle, as it stands, on the host cores: one decode step of the
    same LLaMA-7B-shaped batch (write the 8 new tokens, then attend) over a
    sample of (sequence, head) pairs. Reported in the metric's unit."""
    import numpy as np

    import oracle
    from paged_kv_cache_39_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits = None
        threads = 1
    case = wl.workload(2)
    rows = case.new_token_rows
    old = np.ones(case.key.shape[0], dtype=bool)
    old[rows] = False
    slots_old = np.where(old, case.slot_mapping, -1).astype(np.int32)
    k0, v0 = oracle.write_kv(case.empty_pool(), case.empty_pool(), case.key, case.value,
                             slots_old, case.block_size)
    # the whole batch: 8 sequences x 32 heads
    pairs = [(b, h) for b in range(case.num_seqs) for h in range(case.num_q_heads)]
    steps = 0
    t0 = time.perf_counter()
    while True:   # repeat whole steps until about 10 s of CPU work
        k1, v1 = oracle.write_kv(k0, v0, case.key[rows], case.value[rows],
                                 case.slot_mapping[rows], case.block_size)
        oracle.decode(case.q, k1, v1, case.block_table, case.seq_lens, case.block_size,
                      case.scale, case.dtype, pairs=pairs)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or steps >= 200:
            break
    step_bytes = sum(int(case.seq_lens[b]) for b, _ in pairs) * 2 * case.head_dim * 2
    kv_bytes = steps * step_bytes
    # the same step with the BLAS pool held to one thread (the oracle's
    # Python loops are single-threaded either way)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            s1 = 0
            t1 = time.perf_counter()
            while True:
                k1, v1 = oracle.write_kv(k0, v0, case.key[rows], case.value[rows],
                                         case.slot_mapping[rows], case.block_size)
                oracle.decode(case.q, k1, v1, case.block_table, case.seq_lens, case.block_size,
                              case.scale, case.dtype, pairs=pairs)
                s1 += 1
                d1 = time.perf_counter() - t1
                if d1 >= 5.0 or s1 >= 100:
                    break
        single = {"value": round(s1 * step_bytes / d1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "steps": s1, "seconds": round(d1, 3), "us_per_step": round(d1 / s1 * 1e6, 1)}
    per_config = oracle_per_config()
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": int(threads), "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{steps} full decode steps of the LLaMA-7B-shaped batch, each an oracle "
                      f"KV write of the 8 new tokens then all {len(pairs)} (sequence, head) pairs "
                      f"over 2048 tokens; {dt:.2f} s",
            "us_per_step": round(dt / steps * 1e6, 1),
            "seconds": round(dt, 3),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "single_thread": single,
            "per_config_seconds": per_config}


def oracle_per_config():
    """Wall time of one oracle call per workload (write + attention), on the
    same host threads: tiny decode, ragged GQA decode and packed prefill in
    full; the long-context decode from a sample of (sequence, head) pairs of
    one 131072-token bf16 context, scaled to its 4 x 64 pairs."""
    import numpy as np

    import oracle
    from paged_kv_cache_39_amd import workloads as wl

    res = {}
    for c, key in ((1, "tiny_decode"), (3, "ragged_gqa_decode")):
        case = wl.workload(c)
        t0 = time.perf_counter()
        k, v = oracle.write_kv(case.empty_pool(), case.empty_pool(), case.key, case.value,
                               case.slot_mapping, case.block_size)
        oracle.decode(case.q, k, v, case.block_table, case.seq_lens, case.block_size,
                      case.scale, case.dtype)
        res[key] = round(time.perf_counter() - t0, 3)
    case = wl.workload(4)
    t0 = time.perf_counter()
    k, v = oracle.write_kv(case.empty_pool(), case.empty_pool(), case.key, case.value,
                           case.slot_mapping, case.block_size)
    oracle.varlen(case.q, case.cu_seqlens_q, k, v, case.block_table, case.seq_lens, True,
                  case.block_size, case.dtype)
    res["packed_varlen_prefill"] = round(time.perf_counter() - t0, 3)
    # one sequence of the long-context shape, one kv head: 2 of its 8 query heads
    lc = wl.decode_case(1005, [131072], 8, 1, 128, 128, "bf16", spare=0.0)
    k, v = oracle.write_kv(lc.empty_pool(), lc.empty_pool(), lc.key, lc.value,
                           lc.slot_mapping, lc.block_size)
    t0 = time.perf_counter()
    oracle.decode(lc.q, k, v, lc.block_table, lc.seq_lens, lc.block_size, lc.scale, "bf16",
                  pairs=[(0, 0), (0, 1)])
    per_pair = (time.perf_counter() - t0) / 2
    res["long_context_decode_estimated"] = round(per_pair * 4 * 64, 3)
    res["long_context_decode_note"] = "2 (sequence, head) pairs of one 131072-token context " \
                                      "timed, scaled to the 256 pairs of the call"
    del k, v
    return res


if __name__ == "__main__":
    main()
