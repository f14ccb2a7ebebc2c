#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: for a
decode workload, pa_store_decode (this step's K/V rows stored, and the split-K
partition pass, in one launch -- or the store in a launch of its own when the
batch's grid is larger than the fused kernel keeps resident) -> pa_decode_reduce;
for a prefill workload, pa_store_prefill_varlen (the work-list launch, then the
tile kernel, which reads this step's keys from k/v and stores them).  Inputs are
resident in HBM before timing starts.  Before every step a 1 GiB buffer is read
(outside the timed events) so the 256 MB Infinity Cache and the L2s hold no KV: a
real engine touches 28 layers' caches between two visits to one layer.  The flush
only reads, so it leaves no dirty lines whose write-back would steal bandwidth from
the timed step.

Default workload: the heavy one-layer decode (batch 512, every context 4096, block
256, bf16: 8.59 GB of K/V), the largest single-GPU configuration of the metric.
`value` is its KV read rate: the K and V bytes the step must read (sum of context
lengths x 8 kv heads x 128 x 2 x 2 bytes) over the measured step time.  The line
carries the roofline of the dominant kernel (the decode partition pass) and the
oracle's CPU rate on a bounded sample; under "prefill", the metric's other half:
the Qwen3-0.6B varlen prefill's TFLOP/s with its own MFMA roofline and oracle
baseline; under "also", the batch-64 decode, the shared-prefix decode, the mixed
chunked-prefill step, two-call and layout variants, the q/k norm + rope + store
step, and 28-layer decode steps replayed as HIP graphs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload c4|c2|c3|c5|mixed|p8x2048]
                       [--no-also | --only KEY,...] [--no-cpu-baseline] [--no-prefill-line]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

METRIC = "paged decode KV GB/s and % HBM peak; prefill TFLOP/s (% MFMA), Qwen3-0.6B"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30

WORKLOAD_TEXT = {
    "c2": "Qwen3-0.6B one-layer decode: batch 64, contexts U[128,1024], 16q/8kv heads, d=128, "
          "bf16, block 256, shuffled blocks; store 64 new tokens then decode",
    "c3": "Qwen3-0.6B one-layer varlen causal prefill: 8 sequences, lengths U[64,2048], 3 with "
          "a 256/512-token cached prefix, 16q/8kv, d=128, bf16, block 256; store then prefill",
    "c4": "heavy one-layer decode: batch 512, every context 4096, 16q/8kv, d=128, bf16, "
          "block 256, random block placement",
    "c5": "skewed shared-prefix decode: batch 256, block 16, 192 sequences share a 2048-token "
          "prefix + lognormal tails (median 300, cap 6000), 64 private U[32,8192]",
    "p8x2048": "balanced one-layer varlen causal prefill: 8 fresh prompts of 2048 tokens, "
               "16q/8kv, d=128, bf16, block 256; store then prefill",
    "mixed": "one chunked-prefill engine step through the varlen prefill call: 48 decode rows "
             "(contexts U[128,1024], Lq=1), 4 chunks of 512 after unaligned cached prefixes "
             "U[100,1500], 2 fresh prompts U[64,700]; 16q/8kv, d=128, bf16, block 256",
}


def decode_partition(case):
    """The decode split size the step uses (launch_policy.decode_partition)."""
    from paged_kv_cache_114_amd.launch_policy import decode_partition as policy
    return policy(case.num_seqs, case.num_kv_heads, case.max_context_len)


def prefill_split_keys(case):
    """The prefill key-range size the step uses (launch_policy.prefill_split_keys)."""
    from paged_kv_cache_114_amd.launch_policy import prefill_split_keys as policy
    return policy(case.q_lens, case.context_lens, case.num_q_heads, case.num_kv_heads)


class HipEvents:
    """Timing events from the HIP runtime torch already loaded, created with
    hipEventDisableSystemFence: recording one then costs no system-scope cache
    write-back, which otherwise puts microseconds between the kernels of a step.
    They are recorded on the stream the library launches on."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count):
        import ctypes

        import torch
        torch.cuda.init()
        self.ctypes = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []
        for _ in range(count):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.events.append(e)
        self.stream = torch.cuda.current_stream()

    def record(self, i):
        rc = self.hip.hipEventRecord(self.events[i], self.ctypes.c_void_p(self.stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, i, j):
        """Milliseconds from event i to event j (after a device synchronize)."""
        f = self.ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(self.ctypes.byref(f), self.events[i], self.events[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        for e in getattr(self, "events", []):
            self.hip.hipEventDestroy(e)


class Runner:
    """Buffers and launches for one workload; times each step with HIP events."""

    def __init__(self, name, partition=None, split_keys=None, layout="bshd", case=None,
                 fused_store=True, shared_prefix=False):
        import torch

        import paged_kv_cache_114_amd as pa
        import workloads as W
        self.torch, self.pa, self.W = torch, pa, W
        self.name = name
        self.case = W.FULL_CASES[name]() if case is None else case
        self.vals = W.materialize(self.case, "cuda:0")
        self.layout = layout
        self.fused_store = fused_store
        # decode through pa_decode_shared_prefix: the splits inside a group's shared
        # prefix computed once per group by the MFMA pass
        self.shared_prefix = shared_prefix
        if layout == "bhsd":  # the pool transposed to [NB, Hkv, bs, d]
            for key in ("k_cache", "v_cache"):
                self.vals[key] = self.vals[key].permute(0, 2, 1, 3).contiguous()
        c = self.case
        self.kind = c.kind
        if self.kind == "decode":
            self.partition = partition or decode_partition(c)
            nbytes, self.splits = pa.pa_decode_workspace_size(
                c.num_seqs, c.num_q_heads, c.head_dim, c.max_context_len, self.partition)
            self.ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0")
            self.out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=torch.bfloat16,
                                   device="cuda:0")
        else:
            self.out = torch.empty_like(self.vals["q"])
            self.split_keys = prefill_split_keys(c) if split_keys is None else split_keys
            nbytes, self.splits = pa.pa_prefill_workspace_size(
                c.num_seqs, c.num_new_tokens, c.num_q_heads, c.num_kv_heads, c.head_dim,
                c.max_context_len, self.split_keys)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        self.flush_sink = torch.zeros((), dtype=torch.float32, device="cuda:0")

    def flush(self):
        self.flush_sink.copy_(self.flush_buf.sum())

    def decode_pass(self, kc, vc, fused):
        """The partition pass of one decode step (with this step's store when
        ``fused``) on the pool (kc, vc)."""
        pa, v, c = self.pa, self.vals, self.case
        if self.shared_prefix:
            store = dict(k_new=v["k_new"], v_new=v["v_new"], slot_mapping=v["slot_mapping"])
            pa.pa_decode_shared_prefix(v["q"], kc, vc, v["block_table"], v["context_lens"],
                                       v["prefix_group"], v["prefix_tokens"],
                                       min(int(c.prefix_tokens.max()), c.max_context_len),
                                       c.max_context_len, self.partition, c.scale, self.ws,
                                       layout=self.layout, **(store if fused else {}))
        elif fused:
            pa.pa_store_decode(v["k_new"], v["v_new"], v["slot_mapping"], v["q"], kc, vc,
                               v["block_table"], v["context_lens"], c.max_context_len,
                               self.partition, c.scale, self.ws, layout=self.layout)
        else:
            pa.pa_decode(v["q"], kc, vc, v["block_table"], v["context_lens"], c.max_context_len,
                         self.partition, c.scale, self.ws, layout=self.layout)

    def step(self, ev, k, inner=True):
        """One step; events 4k and 4k+3 bracket it.  With ``inner``, events 4k+1 and
        4k+2 also split it into store, main kernel and (decode) reduce -- each
        record costs a few microseconds of GPU time, so the step itself is timed
        in a pass without them."""
        pa, v, c = self.pa, self.vals, self.case
        mark = ev.record if inner else (lambda i: None)
        ev.record(4 * k)
        fused = self.fused_store
        if not fused:
            pa.pa_store_kv(v["k_new"], v["v_new"], v["k_cache"], v["v_cache"], v["slot_mapping"],
                           layout=self.layout)
        mark(4 * k + 1)
        if self.kind == "decode":  # fused: the store and the partition pass in one launch
            self.decode_pass(v["k_cache"], v["v_cache"], fused)
            mark(4 * k + 2)
            pa.pa_decode_reduce(self.ws, v["context_lens"], self.splits, self.partition,
                                self.out)
        elif self.fused_store:  # the store runs inside the prefill's tile kernel
            pa.pa_store_prefill_varlen(v["k_new"], v["v_new"], v["slot_mapping"], v["q"],
                                       v["k_cache"], v["v_cache"], v["cu_seqlens_q"],
                                       v["cu_seqlens_k"], v["block_table"], c.max_seqlen_q,
                                       c.max_context_len, c.scale, self.out, self.ws,
                                       split_keys=self.split_keys, layout=self.layout)
            mark(4 * k + 2)
        else:
            pa.pa_prefill_varlen(v["q"], v["k_cache"], v["v_cache"], v["cu_seqlens_q"],
                                 v["cu_seqlens_k"], v["block_table"], c.max_seqlen_q,
                                 c.max_context_len, c.scale, self.out, self.ws,
                                 split_keys=self.split_keys, layout=self.layout)
            mark(4 * k + 2)
        ev.record(4 * k + 3)

    def run(self, steps, warmup):
        """Time ``steps`` steps (each after a cache flush, events only around the
        step), then the same number again with events between the kernels for the
        per-kernel split."""
        torch = self.torch
        ev = HipEvents(4 * max(steps, warmup))
        for i in range(warmup):
            self.flush()
            self.step(ev, i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.flush()
            self.step(ev, i, inner=False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = [ev.ms(4 * i, 4 * i + 3) for i in range(steps)]
        for i in range(steps):
            self.flush()
            self.step(ev, i)
        torch.cuda.synchronize()
        store_ms = [ev.ms(4 * i, 4 * i + 1) for i in range(steps)]
        main_ms = [ev.ms(4 * i + 1, 4 * i + 2) for i in range(steps)]
        split_ms = [ev.ms(4 * i, 4 * i + 3) for i in range(steps)]
        return dict(step_ms=sum(step_ms) / steps, store_ms=sum(store_ms) / steps,
                    main_ms=sum(main_ms) / steps, min_step_ms=min(step_ms),
                    step_ms_with_inner_events=sum(split_ms) / steps,
                    wall_ms_per_step=1e3 * wall / steps)

    def store_fused_in_launch(self):
        """Whether pa_store_decode stores inside the partition launch for this batch:
        the library does only when the grid ((sequence, kv head, split) waves) fits
        what the fused kernel keeps resident at once (one 8-wave workgroup per CU at
        these shapes, 2,048 waves on a 256-CU GPU); larger grids store first in a
        launch of their own and run the plain kernel (two workgroups per CU)."""
        c = self.case
        waves = c.num_seqs * c.num_kv_heads * self.splits
        return waves <= 8 * 256

    def partition_events_ms(self, fused=False, reps=10):
        """Average duration of the partition pass alone: HIP events around it in each
        of ``reps`` steps, each after a cache flush (the store, when separate, runs
        before the first event)."""
        torch, pa, v, c = self.torch, self.pa, self.vals, self.case
        ev = HipEvents(2 * reps)
        for r in range(reps):
            self.flush()
            if not fused:
                pa.pa_store_kv(v["k_new"], v["v_new"], v["k_cache"], v["v_cache"],
                               v["slot_mapping"], layout=self.layout)
            ev.record(2 * r)
            self.decode_pass(v["k_cache"], v["v_cache"], fused)
            ev.record(2 * r + 1)
        torch.cuda.synchronize()
        ms = sorted(ev.ms(2 * r, 2 * r + 1) for r in range(reps))
        return ms[len(ms) // 2]

    def main_kernel_amortized(self, layers=16, reps=5, fused=None, planned=False):
        """Average duration of the step's main launch (the fused store + partition
        pass, or the prefill), from HIP events around ``layers`` back-to-back
        launches, each on its own copy of the pool (cold, as in a model's layer
        sweep), after a cache flush: the event records' own cost is spread over
        ``layers`` launches instead of landing on each one."""
        torch, pa, v, c = self.torch, self.pa, self.vals, self.case
        pools = [(v["k_cache"].clone(), v["v_cache"].clone()) for _ in range(layers)]
        if planned:  # the prefill work list built once for all the layers
            pa.pa_prefill_plan(v["cu_seqlens_q"], v["cu_seqlens_k"], c.num_new_tokens,
                               c.num_q_heads, c.num_kv_heads, c.head_dim, c.max_seqlen_q,
                               c.max_context_len, self.ws, split_keys=self.split_keys)
        prefill = pa.pa_prefill_varlen_planned if planned else pa.pa_prefill_varlen
        ev = HipEvents(2 * reps)
        for r in range(reps):
            self.flush()
            ev.record(2 * r)
            for kc, vc in pools:
                if self.kind == "decode":
                    self.decode_pass(kc, vc, self.fused_store if fused is None else fused)
                else:
                    prefill(v["q"], kc, vc, v["cu_seqlens_q"], v["cu_seqlens_k"],
                            v["block_table"], c.max_seqlen_q, c.max_context_len, c.scale,
                            self.out, self.ws, split_keys=self.split_keys, layout=self.layout)
            ev.record(2 * r + 1)
        torch.cuda.synchronize()
        ms = sorted(ev.ms(2 * r, 2 * r + 1) / layers for r in range(reps))
        del pools
        torch.cuda.empty_cache()
        return ms[len(ms) // 2]

    # algorithmic work -------------------------------------------------------------
    def kv_bytes(self):
        return self.case.kv_bytes_logical()

    def store_bytes(self):
        """New K/V rows read and written by the store (fused into the decode launch)."""
        c = self.case
        return c.num_new_tokens * c.num_kv_heads * c.head_dim * c.elt_bytes * 2 * 2

    def prefill_flops(self):
        c = self.case
        return 4 * c.head_dim * c.num_q_heads * c.causal_pairs()

    def summary(self, t):
        c = self.case
        if self.kind == "decode":
            logical = self.kv_bytes()
            unique = c.kv_bytes_unique()
            rate = logical / (t["step_ms"] * 1e-3) / 1e9
            kern = logical / (t["main_ms"] * 1e-3) / 1e9
            out = {"workload": c.name, "layout": self.layout, "fused_store": self.fused_store,
                   "shared_prefix_pass": self.shared_prefix,
                   "kv_GBps_step": round(rate, 1),
                   "decode_kernel_GBps": round(kern, 1),
                   "decode_kernel_frac_hbm": round(kern / HBM_PEAK_GBS, 4),
                   "ms_per_step": round(t["step_ms"], 5),
                   "decode_kernel_ms": round(t["main_ms"], 5),
                   "partition_tokens": self.partition, "num_splits": self.splits}
            if unique != logical:
                out["unique_kv_GBps_kernel"] = round(unique / (t["main_ms"] * 1e-3) / 1e9, 1)
                out["unique_frac_hbm"] = round(unique / (t["main_ms"] * 1e-3) / 1e9 /
                                               HBM_PEAK_GBS, 4)
            return out
        flops = self.prefill_flops()
        tf = flops / (t["main_ms"] * 1e-3) / 1e12
        return {"workload": c.name, "layout": self.layout, "fused_store": self.fused_store,
                "prefill_TFLOPs_kernel": round(tf, 2),
                "frac_bf16_mfma": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                "ms_per_step": round(t["step_ms"], 5), "prefill_kernel_ms": round(t["main_ms"], 5),
                "gflop": round(flops / 1e9, 3), "split_keys": self.split_keys,
                "num_splits": self.splits}


KERNEL_SOURCES = {
    "decode_partition_kernel": ["paged_kv_cache_114_amd/csrc/pa_decode.hip",
                                "paged_kv_cache_114_amd/csrc/pa_common.h"],
    "prefix_split_kernel": ["paged_kv_cache_114_amd/csrc/pa_prefix.hip",
                            "paged_kv_cache_114_amd/csrc/pa_store_rows.h",
                            "paged_kv_cache_114_amd/csrc/pa_common.h"],
    "prefill_kernel": ["paged_kv_cache_114_amd/csrc/pa_prefill.hip",
                       "paged_kv_cache_114_amd/csrc/pa_common.h"],
}


def measured_traffic(workload, kernel):
    """HBM bytes per launch (read + written) from the committed FETCH_SIZE / WRITE_SIZE
    profile, or None when there is none or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel.removesuffix("_plain").removesuffix("_store")]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    with open(path) as fh:
        rec = json.load(fh)
    for e in rec["entries"]:
        if e["workload"] == workload and e["kernel"] == kernel and e["source_hash"] == digest:
            return int(round(e["read_bytes"] + e["write_bytes"]))
    return None


_SHARED = {}


def _oracle_worker_init(root, shm_name, pool_shape, pool_dtype, meta):
    """Worker processes import only NumPy and the oracle (never torch or HIP); they see
    the host copy of the K/V pools through shared memory and the rest as plain arrays."""
    from multiprocessing import shared_memory

    import numpy as np
    if root not in sys.path:
        sys.path.insert(0, root)
    shm = shared_memory.SharedMemory(name=shm_name)
    pools = np.ndarray((2,) + tuple(pool_shape), dtype=pool_dtype, buffer=shm.buf)
    _SHARED.update(meta, shm=shm, k_cache=pools[0], v_cache=pools[1])


def _oracle_task(seqs):
    """Gather one chunk of sequences (their blocks packed into a compact pool, as the
    single-core sample does) and time store + attention with the fp64 oracle."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    d = _SHARED
    bs = d["block_size"]
    used = sorted({int(p) for b in seqs
                   for p in d["block_table"][b, :-(-int(d["context_lens"][b]) // bs)]})
    remap = {p: i for i, p in enumerate(used)}
    packed = d["g2p"][used]  # the shared pools hold only the sampled sequences' blocks
    kc = d["k_cache"][packed]
    vc = d["v_cache"][packed]
    bt = np.full((len(seqs), d["block_table"].shape[1]), -1, np.int32)
    for r, b in enumerate(seqs):
        n = -(-int(d["context_lens"][b]) // bs)
        bt[r, :n] = [remap[int(p)] for p in d["block_table"][b, :n]]
    rows = [i for i, s in enumerate(d["new_seq"].tolist()) if s in set(seqs)]
    slots = d["slot_mapping"][rows].astype(np.int64)
    slot_map = np.array([remap[int(x) // bs] * bs + int(x) % bs for x in slots], np.int64)
    q = d["q"][seqs] if d["kind"] == "decode" else d["q"][rows]
    ctx = d["context_lens"][seqs]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kst, vst = oracle.store(kc, vc, d["k_new"][rows], d["v_new"][rows], slot_map)
        if d["kind"] == "decode":
            oracle.decode(q, kst, vst, bt, ctx, d["scale"], d["dtype"])
        else:
            q_lens = ctx - d["num_cached"][seqs]
            cu_q = np.concatenate([[0], np.cumsum(q_lens)])
            cu_k = np.concatenate([[0], np.cumsum(ctx)])
            oracle.prefill(q, kst, vst, cu_q, cu_k, bt, d["scale"], d["dtype"])
        return time.perf_counter() - t0


def cpu_baseline(name, budget_s=12.0, all_cores_s=8.0):
    """The oracle, untuned, on host copies of the same inputs: store + attention
    over the workload's sequences (in a fixed random order, passing over them again
    while time is left) until about budget_s seconds of oracle time."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import workloads as W
    from pa_runner import HostInputs

    case = W.FULL_CASES[name]()
    vals = W.materialize(case, "cuda:0")
    perm = [int(b) for b in np.random.default_rng(0).permutation(case.num_seqs)]
    order = list(perm)
    done, elapsed, work, passes = [], 0.0, 0, 1
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            if not order:
                order, passes = list(perm), passes + 1
            chunk = [int(order.pop()) for _ in range(min(4, len(order)))]
            host = HostInputs(case, vals, chunk)
            t0 = time.perf_counter()
            if case.kind == "decode":
                host.decode()
            else:
                host.prefill()
            elapsed += time.perf_counter() - t0
            done += chunk
    c = case
    if case.kind == "decode":
        work = 2 * c.num_kv_heads * c.head_dim * c.elt_bytes * int(c.context_lens[done].sum())
        value, unit = work / elapsed / 1e9, "GB/s"
    else:
        pairs = 0
        for b in done:
            lq, lk = int(c.q_lens[b]), int(c.context_lens[b])
            pairs += lq * (lk - lq + 1) + lq * (lq - 1) // 2
        value, unit = 4 * c.head_dim * c.num_q_heads * pairs / elapsed / 1e12, "TFLOP/s"
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass

    # The same oracle on every host core: spawned processes (they never touch the GPU),
    # one BLAS thread each, over chunks of 4 sequences cycling through the same order,
    # sized from the single-core rate to last about all_cores_s seconds of wall time.
    all_cores = None
    if all_cores_s > 0:
        import concurrent.futures as cf
        import multiprocessing as mp
        from multiprocessing import shared_memory
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        per_task = elapsed / max(1, -(-len(done) // 4))
        n_tasks = int(min(40000, max(workers, all_cores_s * workers / max(per_task, 1e-4))))
        # the workers cycle over the sequences whose blocks fit 2 GiB of shared memory
        bs = c.block_size
        block_bytes = 2 * c.block_size * c.num_kv_heads * c.head_dim * c.elt_bytes
        subset, blocks = [], set()
        for b in perm:
            mine = set(int(x) for x in c.block_table[b, :-(-int(c.context_lens[b]) // bs)])
            if subset and len(blocks | mine) * block_bytes > (2 << 30):
                break
            subset.append(b)
            blocks |= mine
        used_g = sorted(blocks)
        g2p = np.full(c.num_blocks, -1, np.int64)
        g2p[used_g] = np.arange(len(used_g))
        chunks = [[subset[(4 * t + i) % len(subset)] for i in range(4)] for t in range(n_tasks)]
        idx = torch.tensor(used_g, dtype=torch.long, device="cuda:0")
        kraw = W.raw_numpy(vals["k_cache"].index_select(0, idx), c.dtype)
        shm = shared_memory.SharedMemory(create=True, size=2 * kraw.nbytes)
        try:
            pools = np.ndarray((2,) + kraw.shape, dtype=kraw.dtype, buffer=shm.buf)
            pools[0] = kraw
            pools[1] = W.raw_numpy(vals["v_cache"].index_select(0, idx), c.dtype)
            del kraw
            meta = {"block_size": c.block_size, "block_table": c.block_table, "g2p": g2p,
                    "context_lens": c.context_lens, "num_cached": c.num_cached,
                    "new_seq": c.new_seq, "slot_mapping": c.slot_mapping,
                    "k_new": W.raw_numpy(vals["k_new"], c.dtype),
                    "v_new": W.raw_numpy(vals["v_new"], c.dtype),
                    "q": W.raw_numpy(vals["q"], c.dtype), "scale": c.scale, "dtype": c.dtype,
                    "kind": c.kind}
            root = os.path.dirname(os.path.abspath(__file__))
            with cf.ProcessPoolExecutor(
                    max_workers=workers, mp_context=mp.get_context("spawn"),
                    initializer=_oracle_worker_init,
                    initargs=(root, shm.name, pools.shape[1:], pools.dtype, meta)) as pool:
                list(pool.map(_oracle_task, chunks[:workers]))  # start-up, not timed
                t0 = time.perf_counter()
                list(pool.map(_oracle_task, chunks, chunksize=1))
                wall = time.perf_counter() - t0
            del pools
        finally:
            shm.close()
            shm.unlink()
        seqs_done = [b for ch in chunks for b in ch]
        if case.kind == "decode":
            w_all = 2 * c.num_kv_heads * c.head_dim * c.elt_bytes * int(
                c.context_lens[seqs_done].sum())
            v_all = w_all / wall / 1e9
        else:
            pairs = sum(int(c.q_lens[b]) * (int(c.context_lens[b]) - int(c.q_lens[b]) + 1) +
                        int(c.q_lens[b]) * (int(c.q_lens[b]) - 1) // 2 for b in seqs_done)
            v_all = 4 * c.head_dim * c.num_q_heads * pairs / wall / 1e12
        all_cores = {"value": round(v_all, 4), "unit": unit, "cores": workers,
                     "sample": f"{len(seqs_done)} sequence evaluations in {len(chunks)} tasks of "
                               f"4 sequences (cycling over {len(subset)} of the "
                               f"{c.num_seqs} sequences) on {workers} worker processes (1 BLAS "
                               f"thread each, their blocks shared read-only)",
                     "seconds": round(wall, 2)}
    return {"value": round(value, 4), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} sequence evaluations over {passes} pass(es) of the "
                      f"{c.num_seqs} sequences of {c.name} (store + attention, fp64 NumPy, "
                      f"1 BLAS thread), {elapsed:.1f} s of oracle time",
            "cpu": cpu, "seconds": round(elapsed, 2), "all_cores": all_cores}


def main_is_decode(name):
    import workloads as W
    return W.FULL_CASES[name]().kind == "decode"


def roofline(run, t, name):
    """The step's rate (``value``) and the roofline block of its dominant kernel.

    Decode: the partition pass (HBM-bound); its launch duration comes from HIP
    events around 16 back-to-back launches on 16 pool copies after a cache flush
    when 16 copies fit in 24 GiB, else from events around the pass in each step
    (C4: 1.4 ms a launch, so the events' few microseconds do not matter).  When the
    library stores this step's rows in their own launch (a grid larger than the
    fused kernel keeps resident, as for 512 sequences), the pass timed is the
    plain partition kernel and its bytes are the KV read only.
    Prefill: the pa_prefill_varlen call, i.e. the work-list kernel and the tile
    kernel (MFMA-bound), timed the same way."""
    pool_bytes = 2 * run.vals["k_cache"].numel() * run.vals["k_cache"].element_size()
    amortize = pool_bytes * 16 < (24 << 30)
    traffic_note = ("HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE "
                    "profile of the same kernel source (profiles/hbm_traffic.json); null when the "
                    "source changed since")
    if run.kind == "decode":
        # pa_decode_shared_prefix stores in its prefix pass's launch whatever the grid;
        # pa_store_decode stores in the partition launch when the fused kernel keeps the
        # grid resident, else in a launch of its own before it
        fused_launch = run.fused_store and (run.shared_prefix or run.store_fused_in_launch())
        if amortize:
            kernel_ms = run.main_kernel_amortized(fused=fused_launch)
            timing = ("HIP events around 16 back-to-back launches on 16 pool copies after a "
                      "cache flush, divided by 16")
        else:
            kernel_ms = run.partition_events_ms(fused=fused_launch)
            timing = "HIP events around the partition pass in each step (after a cache flush)"
        value = run.kv_bytes() / (t["step_ms"] * 1e-3) / 1e9
        kname = "decode_partition_kernel"
        if run.shared_prefix:
            # the prefix pass reads each group's shared blocks once and the partition
            # pass the rest: together every K/V byte once (the unique bytes)
            alg = run.case.kv_bytes_unique() + (run.store_bytes() if fused_launch else 0)
            # the two launches' counted bytes (the profile keys this path "<workload>s")
            parts = [measured_traffic(name + "s", k)
                     for k in ("prefix_split_kernel", kname + "_plain")]
            traffic = None if None in parts else sum(parts)
            kdesc = ("pa_decode_shared_prefix: prefix_split_kernel (the prefix splits" +
                     (", this step's store" if fused_launch else "") +
                     " and the partition pass's work list) + " + kname + " (plain)")
        else:
            alg = run.kv_bytes() + (run.store_bytes() if fused_launch else 0)
            traffic = measured_traffic(name, kname + ("" if fused_launch else "_plain"))
            kdesc = kname + (" (with the fused store)" if fused_launch else
                             " (plain; this step stores its rows in a launch of its own)")
        achieved = alg / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "traffic_source": traffic_note,
                "algorithmic_bytes": alg, "kernel": kdesc,
                "kernel_ms": round(kernel_ms, 5), "kernel_ms_timing": timing}
        return value, "GB/s", roof
    kernel_ms = run.main_kernel_amortized()
    value = run.prefill_flops() / (t["step_ms"] * 1e-3) / 1e12
    achieved = run.prefill_flops() / (kernel_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(name, "prefill_kernel"), "traffic_source": traffic_note,
            "algorithmic_flops": run.prefill_flops(),
            "kernel": "pa_prefill_varlen: prefill_plan_kernel + prefill_kernel (tile kernel)",
            "kernel_ms": round(kernel_ms, 5),
            "kernel_ms_timing": ("HIP events around 16 back-to-back calls on 16 pool copies "
                                 "after a cache flush, divided by 16")}
    # an engine builds the work list once per step for all its layers (pa_prefill_plan)
    planned_ms = run.main_kernel_amortized(planned=True)
    roof["planned_call_ms"] = round(planned_ms, 5)
    roof["planned_call_frac"] = round(run.prefill_flops() / (planned_ms * 1e-3) / 1e12 /
                                      BF16_MFMA_PEAK_TFLOPS, 4)
    roof["planned_call_timing"] = ("the same 16 calls through pa_prefill_varlen_planned on one "
                                   "work list built before them (the layers of one step)")
    return value, "TFLOP/s", roof


def graph_decode(name="c2", layers=28, steps=20, warmup=3, partition=None, batch=None,
                 fused=False):
    """A decode step of a layers-deep model at one workload's shapes: per layer,
    the store fused into the partition pass, then the reduce, on that layer's
    own cache, all on one stream.  Timed eager and as one captured HIP graph
    replay.  ``fused``: the store is the q/k norm + rope + store step on the
    layer's projection rows, then the partition pass reads the rotated Q it
    writes (3 launches per layer)."""
    import torch

    import paged_kv_cache_114_amd as pa
    import workloads as W
    case = W.FULL_CASES[name]() if batch is None else W.c2_decode(
        batch=batch, name=f"c2_decode_b{batch}")
    base = W.materialize(case, "cuda:0")
    p = partition or decode_partition(case)
    nbytes, splits = pa.pa_decode_workspace_size(case.num_seqs, case.num_q_heads, case.head_dim,
                                                 case.max_context_len, p)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0")
    proj = W.projection_inputs(case, "cuda:0") if fused else {}
    hq, hkv = case.num_q_heads, case.num_kv_heads
    lays = []
    for _ in range(layers):
        lays.append(dict(base, k_cache=base["k_cache"].clone(), v_cache=base["v_cache"].clone(),
                         out=torch.empty_like(base["q"]), q_rot=torch.empty_like(base["q"])))

    def step():
        for lay in lays:
            if fused:
                pa.pa_qk_norm_rope_store(proj["qkv"], proj["q_norm_weight"],
                                         proj["k_norm_weight"], proj["positions"],
                                         proj["slot_mapping"], hq, hkv, 1e-6, 1e6, lay["q_rot"],
                                         lay["k_cache"], lay["v_cache"])
                pa.pa_decode(lay["q_rot"], lay["k_cache"], lay["v_cache"], lay["block_table"],
                             lay["context_lens"], case.max_context_len, p, case.scale, ws)
            else:
                pa.pa_store_decode(lay["k_new"], lay["v_new"], lay["slot_mapping"], lay["q"],
                                   lay["k_cache"], lay["v_cache"], lay["block_table"],
                                   lay["context_lens"], case.max_context_len, p, case.scale, ws)
            pa.pa_decode_reduce(ws, lay["context_lens"], splits, p, lay["out"])

    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros((), dtype=torch.float32, device="cuda:0")

    def timed(fn):
        ev = HipEvents(2 * (steps + warmup))
        for i in range(warmup + steps):
            sink.copy_(flush_buf.sum())
            ev.record(2 * i)
            fn()
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        return sum(ev.ms(2 * i, 2 * i + 1) for i in range(warmup, warmup + steps)) / steps

    eager_ms = timed(step)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_ms = timed(graph.replay)
    kv = layers * case.kv_bytes_logical()
    per_layer = ("q/k norm + rope + store, decode, reduce" if fused
                 else "store fused into decode, reduce")
    return {"workload": f"{case.name} x {layers} layers ({per_layer} per layer)",
            "layers": layers, "launches_per_step": (3 if fused else 2) * layers,
            "eager_ms_per_step": round(eager_ms, 4), "graph_ms_per_step": round(graph_ms, 4),
            "graph_speedup": round(eager_ms / graph_ms, 3),
            "kv_GBps_graph": round(kv / (graph_ms * 1e-3) / 1e9, 1),
            "kv_GBps_eager": round(kv / (eager_ms * 1e-3) / 1e9, 1),
            "partition_tokens": p}


def norm_rope_store(name, steps=15, warmup=3):
    """The per-head q/k RMSNorm + RoPE + paged store step over one workload's new
    tokens (its fused projection rows), timed alone with HIP events after a
    cache flush.  Algorithmic bytes per token: the projection row read once
    ((Hq + 2 Hkv) d elements) and written once (Q to q_out, K and V to the
    cache), plus its position and slot (8 bytes)."""
    import torch

    import paged_kv_cache_114_amd as pa
    import workloads as W
    case = W.FULL_CASES[name]()
    vals = W.materialize(case, "cuda:0")
    inp = W.projection_inputs(case, "cuda:0")
    t, hq, hkv, d = case.num_new_tokens, case.num_q_heads, case.num_kv_heads, case.head_dim
    q_out = torch.empty((t, hq, d), dtype=inp["qkv"].dtype, device="cuda:0")
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros((), dtype=torch.float32, device="cuda:0")
    ev = HipEvents(2 * (steps + warmup))
    for i in range(warmup + steps):
        sink.copy_(flush_buf.sum())
        ev.record(2 * i)
        pa.pa_qk_norm_rope_store(inp["qkv"], inp["q_norm_weight"], inp["k_norm_weight"],
                                 inp["positions"], inp["slot_mapping"], hq, hkv, 1e-6, 1e6,
                                 q_out, vals["k_cache"], vals["v_cache"])
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ms = sum(ev.ms(2 * i, 2 * i + 1) for i in range(warmup, warmup + steps)) / steps
    nbytes = t * (2 * (hq + 2 * hkv) * d * case.elt_bytes + 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{case.name} new tokens (q/k norm + rope + store)", "tokens": t,
            "kernel_ms": round(ms, 5), "algorithmic_bytes": nbytes, "GBps": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--partition", type=int, default=None,
                    help="decode split size in tokens (default: chosen from the workload)")
    ap.add_argument("--split-keys", type=int, default=None,
                    help="prefill keys per workgroup for long query tiles (0: no split; "
                         "default: chosen from the workload)")
    ap.add_argument("--no-also", action="store_true", help="skip the other workloads")
    ap.add_argument("--only", default=None,
                    help="comma-separated keys of the 'also' entries to run (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode through pa_decode_shared_prefix (the workload's prefix groups)")
    ap.add_argument("--no-prefill-line", action="store_true",
                    help="skip the C3 prefill roofline and oracle block of a decode headline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run plain device copies of this size (a known-traffic kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(decode shards by sequence or kv head with no exchange; see the "
                         "design notes). Run with --gpus 1.\n")
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": args.steps}), flush=True)
        return

    main_run = Runner(args.workload, args.partition, args.split_keys,
                      shared_prefix=args.shared_prefix)
    t = main_run.run(args.steps, args.warmup)
    summ = main_run.summary(t)
    c = main_run.case
    value, unit, roof = roofline(main_run, t, args.workload)
    del main_run
    torch.cuda.empty_cache()

    # The metric's second half: the varlen prefill's TFLOP/s against the bf16 MFMA
    # peak, on the Qwen3-0.6B varlen batch, with the oracle beside it.
    prefill_line = None
    if main_is_decode(args.workload) and not args.no_prefill_line:
        pr = Runner("c3")
        tp = pr.run(max(5, args.steps // 2), 3)
        p_value, p_unit, p_roof = roofline(pr, tp, "c3")
        prefill_line = {"workload": WORKLOAD_TEXT["c3"], "value": round(p_value, 2),
                        "unit": p_unit, "ms_per_step": round(tp["step_ms"], 5),
                        "roofline": p_roof, "detail": pr.summary(tp)}
        del pr
        torch.cuda.empty_cache()

    also = {}
    only = set(args.only.split(",")) if args.only else None
    if not args.no_also:
        for name in ("c2", "c4", "c5", "c3", "mixed"):
            if name == args.workload or (only and name not in only):
                continue
            try:
                # C5's sequences share prefix blocks: its step declares the groups
                r = Runner(name, shared_prefix=name == "c5")
                also[name] = r.summary(r.run(max(5, args.steps // 2), 3))
                del r
                torch.cuda.empty_cache()
            except Exception as e:  # a workload whose kernel is missing is reported as such
                also[name] = {"error": f"{type(e).__name__}: {e}"}
        # the two-call store + decode, the head-major pool, and smaller blocks
        import workloads as W
        # C5 through pa_store_decode, its prefix groups not declared: every member
        # reads the shared blocks itself
        for key in ("c5_prefix_undeclared",):
            if only and key not in only:
                continue
            try:
                r = Runner("c5")
                also[key] = r.summary(r.run(max(5, args.steps // 2), 3))
                del r
                torch.cuda.empty_cache()
            except Exception as e:
                also[key] = {"error": f"{type(e).__name__}: {e}"}
        variants = [("c2_two_call", "c2", "bshd", None, False),
                    ("c4_two_call", "c4", "bshd", None, False),
                    ("c3_two_call", "c3", "bshd", None, False),
                    ("layout_bhsd_c2", "c2", "bhsd", None, True),
                    ("layout_bhsd_c3", "c3", "bhsd", None, True)]
        for bs in (16, 64):
            for layout in ("bshd", "bhsd"):
                variants.append((f"bs{bs}_{layout}_c2", "c2", layout,
                                 W.c2_decode(name=f"c2_decode_b64_bs{bs}", bs=bs), True))
        for key, name, layout, case, fused in variants:
            if only and key not in only:
                continue
            try:
                r = Runner(name, layout=layout, case=case, fused_store=fused)
                also[key] = r.summary(r.run(max(5, args.steps // 2), 3))
                also[key]["block_size"] = r.case.block_size
                del r
                torch.cuda.empty_cache()
            except Exception as e:
                also[key] = {"error": f"{type(e).__name__}: {e}"}
        for name in ("c2", "c3", "mixed"):
            if only and f"norm_rope_store_{name}" not in only:
                continue
            try:
                also[f"norm_rope_store_{name}"] = norm_rope_store(name, max(5, args.steps // 2))
                torch.cuda.empty_cache()
            except Exception as e:
                also[f"norm_rope_store_{name}"] = {"error": f"{type(e).__name__}: {e}"}
        for key, batch, fused in (("c2_graph28", None, False), ("c2_b16_graph28", 16, False),
                                  ("c2_b4_graph28", 4, False), ("c2_b1_graph28", 1, False),
                                  ("c2_graph28_fused_rope", None, True)):
            if only and key not in only:
                continue
            try:
                also[key] = graph_decode("c2", 28, steps=max(5, args.steps // 2), batch=batch,
                                         fused=fused)
                torch.cuda.empty_cache()
            except Exception as e:
                also[key] = {"error": f"{type(e).__name__}: {e}"}

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["step_ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, random block placement)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "case": c.name,
                   "batch": c.num_seqs, "max_context": c.max_context_len,
                   "block_size": c.block_size, "q_heads": c.num_q_heads,
                   "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "parallelism": "single GPU"},
        "timing": {"store_ms": round(t["store_ms"], 5), "main_kernel_ms": round(t["main_ms"], 5),
                   "min_step_ms": round(t["min_step_ms"], 5),
                   "step_ms_with_inner_events": round(t["step_ms_with_inner_events"], 5),
                   "wall_ms_per_step_incl_cache_flush": round(t["wall_ms_per_step"], 4)},
        "roofline": roof,
        "detail": summ,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    if prefill_line is not None:
        line["prefill"] = prefill_line
        if not args.no_cpu_baseline:
            line["prefill"]["cpu_baseline"] = cpu_baseline("c3", budget_s=8.0, all_cores_s=6.0)
    line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
