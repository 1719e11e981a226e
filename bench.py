"""Benchmark: one paged decode step of an OPT-13B-shaped attention layer on one GPU.

A step is the whole hot path over one batch: the host allocator reserves one
slot per request (copy-on-write pairs, if any, are copied), the new tokens'
K/V are written into their slots, block tables are uploaded, and decode
attention runs over every request's context through its block table.  Inputs
(pools, queries, new tokens) are resident in HBM before timing starts.

Prints one JSON line.  ``value`` is algorithmic KV bytes read by decode
attention per step (logical tokens only: sum(L) * 2 * Hkv * D * 2 B) divided
by the wall time per step; ``roofline`` is the same byte count per decode
divided by the decode launches' duration: kernel-level HIP events (the first
kernel's start to the last kernel's end, recorded by the launches themselves on
the launch stream) on every 5th timed step.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of requests.

    python bench.py [--steps K] [--warmup W] [--workload opt13b|gqa|long_context]

Other workloads: ``prefill`` (prompt-phase attention, FLOP/s against the fp16
matrix peak), ``swap`` (requests moved to the pinned host tier and back, GB/s
against the host link) and ``beams`` (beam-search-like fork / cancel churn with
copy-on-write, tokens/s with the decode roofline on unique bytes).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GPU_INFO = None                             # amd-smi summary, filled in by main()
METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + µs/step, OPT-13B shape"


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; parallel_sampling: its 128 steps)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="opt13b",
                    choices=["opt13b", "gqa", "long_context", "parallel_sampling", "tiny", "prefill",
                             "swap", "beams"])
    ap.add_argument("--partition", default="auto",
                    help="tokens per split-context partition, 0 = one pass, or 'auto'")
    ap.add_argument("--block-size", type=int, default=0,
                    help="decode workloads: store the same requests and values in blocks of this "
                         "many tokens (8, 16, 32, 64 or 128; 0 = the workload's own, 16); the "
                         "long-context workload is stated as a sweep over all five")
    ap.add_argument("--kernel-policy", default="default", choices=["default", "valu"],
                    help="head-group kernel: MFMA (default for fp16 groups of >= 4) or VALU")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only measure the HBM read ceiling (pkv_read_probe) and exit")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the read-ceiling measurement that the decode line reports")
    ap.add_argument("--timeline", action="store_true",
                    help="opt13b, gqa, long_context, tiny: run on the instrumented "
                         "libpagedkv_timeline.so (python -m paged_kv_cache_244_amd.build "
                         "--timeline), record the per-wave timeline of the decode launch of "
                         "one step after the warmup and print its summary (no JSON line)")
    ap.add_argument("--time-every", type=int, default=5,
                    help="decode, beams and prefill workloads: the attention launches of every "
                         "n-th timed step take "
                         "kernel-level timing events (first kernel's start to last kernel's "
                         "end); timed launches cost the GPU several microseconds more, so "
                         "timing every step would slow the steps being measured")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough budget for the CPU oracle baseline (0 disables it)")
    ap.add_argument("--layout", default="paged", choices=["paged", "contiguous"],
                    help="K/V layout: the paged pool (the product path) or one contiguous row "
                         "per (request, KV head) without a block table, for comparison")
    ap.add_argument("--no-prefix-groups", action="store_true",
                    help="parallel_sampling and beams: read shared prompt blocks once per "
                         "request instead of once per group (for comparison)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool replicas rotated over the steps, as a model's layers would be "
                         "(0 = enough for 2 GiB of K/V pools, so no step finds its pool in the "
                         "256 MiB last-level cache)")
    return ap.parse_args()


def kv_bytes(lengths, w):
    return int(np.sum(lengths, dtype=np.int64)) * 2 * w.num_kv_heads * w.head_dim * 2


def counter_traffic(workload_name, kernel="pa_decode"):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary,
    or None when there is none for this workload or the kernel source changed since."""
    import hashlib
    import re

    stem = kernel if workload_name is None else f"{kernel}_{workload_name}"
    path = os.path.join(ROOT, "profiles", f"{stem}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    for rel, digest in rec["kernel_sources_sha256"].items():
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
            return None
    return rec


def cpu_baseline(w, budget_s):
    """Time the oracle's paged attention on a sample of requests, single-threaded BLAS."""
    from threadpoolctl import threadpool_limits

    from oracle import alloc_model, attention, cache

    order = np.argsort(np.random.default_rng(0).random(w.num_seqs))
    # Estimate the oracle's rate on a small request, then take requests until ~budget.
    picked, tokens = [], 0
    est_tok_per_s = 25_000.0 * (40 * 128) / (w.num_q_heads * w.head_dim)
    for i in order:
        picked.append(int(i))
        tokens += int(w.lengths[i])
        if tokens / est_tok_per_s >= budget_s:
            break
    lens = w.lengths[picked]
    nb_need = int(sum(-(-int(L) // w.block_size) for L in lens))
    m = alloc_model.AllocatorModel(nb_need, w.block_size)
    shape = (nb_need, w.num_kv_heads, w.block_size, w.head_dim)
    kp = np.zeros(shape, dtype=np.float16)
    vp = np.zeros(shape, dtype=np.float16)
    seqs = []
    for i in picked:
        s = m.create()
        seqs.append(s)
        k, v = w.tokens(i)
        slots, _ = m.append(s, len(k))
        cache.write_slots(kp, vp, k, v, slots, w.block_size)
    max_blocks = max(len(m.table(s)) for s in seqs)
    tables, lens_l = m.export(seqs, max_blocks, 0)
    q = w.q[picked]
    # Whole passes over the sample until about the budget has been spent (at least one).
    passes, dt = 0, 0.0
    with threadpool_limits(limits=1):
        while passes == 0 or dt < 0.8 * budget_s:
            t0 = time.perf_counter()
            attention.attend_paged(q, kp, vp, np.array(tables), lens_l, w.block_size, w.scale)
            dt += time.perf_counter() - t0
            passes += 1
    nbytes = kv_bytes(lens, w) * passes
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(picked)} of {w.num_seqs} requests ({int(lens.sum())} tokens) x {passes} "
                      f"passes, fp64 numpy attend_paged, attention only, {dt:.1f} s",
            "seconds": round(dt, 2), "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "threads": 1}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_info():
    """Device name, partition modes and clock limits from amd-smi (child processes, read
    only), or None where the tool is missing or says nothing usable.  Skipped under
    rocprofv3 (it exports ROCPROF_OUTPUT_PATH): the profiler's library would start in each
    child, and the amd-smi launcher replaces itself through /usr/bin/env."""
    import subprocess

    if "ROCPROF_OUTPUT_PATH" in os.environ:
        return None

    def query(args):
        try:
            r = subprocess.run(["amd-smi"] + args + ["-g", "0", "--json"], capture_output=True,
                               text=True, timeout=30)
            return json.loads(r.stdout)["gpu_data"][0] if r.returncode == 0 else None
        except (OSError, ValueError, KeyError, IndexError, subprocess.SubprocessError):
            return None

    info = {}
    st = query(["static"])
    if st:
        info["name"] = st.get("asic", {}).get("market_name")
    pt = query(["static", "--partition"])
    if pt and isinstance(pt.get("partition"), dict):
        part = pt["partition"]
        info["partition"] = f"{part.get('accelerator_partition')}/{part.get('memory_partition')}"
    ck = query(["metric", "--clock"])
    if ck:
        clock = ck.get("clock", {})
        gfx = clock.get("gfx_0", {}).get("max_clk", {})
        mem = clock.get("mem_0", {}).get("clk", {})
        info["gfx_max_mhz"] = gfx.get("value") if isinstance(gfx, dict) else None
        info["mem_mhz"] = mem.get("value") if isinstance(mem, dict) else None
    return info or None


def copy_probe():
    """A plain device-to-device copy of known size, to calibrate HBM byte counters."""
    import torch

    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "kernel": "elementwise copy (torch copy_)"}), flush=True)


def kernel_timers(n):
    """n library-made event pairs for kernel-level timing (``_lib.time_next_call``)."""
    from paged_kv_cache_244_amd import _lib
    return [_lib.KernelTimer() for _ in range(n)]


class TimingRing:
    """Timing events in a small ring.  The HIP runtime slowed the steps of a run
    measurably (1.27 -> 1.9-2.6 ms per prefill step on MI355X) once 60-100 events
    were alive in the process, whether recorded or not, so a run keeps ``size``
    event sets and reads each one's result just before reusing it (by then its
    step finished long ago).  ``take(key)`` returns the set to use for ``key``;
    ``results()`` returns {key: read(set)} for every key taken."""

    def __init__(self, size, make, read):
        self.slots = [[None, make()] for _ in range(size)]
        self.n, self.read, self.out = 0, read, {}

    def take(self, key):
        slot = self.slots[self.n % len(self.slots)]
        self.n += 1
        if slot[0] is not None:
            self.out[slot[0]] = self.read(slot[1])
        slot[0] = key
        return slot[1]

    def results(self):
        for slot in self.slots:
            if slot[0] is not None:
                self.out[slot[0]] = self.read(slot[1])
                slot[0] = None
        return self.out


def timer_ring(size=8):
    """Library-made events taking a call's kernel start and end."""
    from paged_kv_cache_244_amd import _lib

    return TimingRing(size, _lib.KernelTimer, lambda t: t.ms())


PROBE_TILE_BYTES = 4096


def read_ceiling(dev, nbytes=4 << 30, reps=5):
    """HBM read bandwidth of the library's plain read kernel (pkv_read_probe) over a
    4 GiB buffer (16x the last-level cache), in order and as 4 KiB tiles gathered in
    a seeded random order (the access pattern of a paged pool); the best of a few
    grid sizes, median of ``reps`` launches each, timed by the kernel's own start
    and end events (``_lib.time_next_call``) on the launch stream."""
    import torch

    from paged_kv_cache_244_amd import _lib

    num_tiles = nbytes // PROBE_TILE_BYTES
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.zero_()
    perm = torch.randperm(num_tiles, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    order = perm.to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    result = {}
    for mode, order_ptr in (("sequential", None), ("tile_gather", order.data_ptr())):
        best = None
        for wgs in (1024, 2048, 4096):
            ms = []
            for t in kernel_timers(reps + 1):
                _lib.time_next_call(t)
                _lib._check(_lib.lib().pkv_read_probe(buf.data_ptr(), num_tiles, order_ptr,
                                                      sink.data_ptr(), wgs, stream.cuda_stream))
                ms.append(t.ms())
            gbs = nbytes / (float(np.median(ms[1:])) / 1e3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, wgs, float(np.median(ms[1:])))
        result[mode] = {"gbs": round(best[0], 1), "workgroups": best[1],
                        "us": round(best[2] * 1e3, 1)}
    del buf, order
    torch.cuda.empty_cache()
    result["bytes"] = nbytes
    result["kernel"] = "pkv_read_probe (read_probe_kernel)"
    return result


def stream_probe():
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(json.dumps({"read_ceiling": read_ceiling(dev), "gpu": GPU_INFO}), flush=True)


REPLICA_TARGET_BYTES = 2 << 30


def replicas_for(num_blocks, w, requested):
    """Pool replicas so that the rotated K/V pools total at least 2 GiB (at most 16)."""
    if requested > 0:
        return requested
    pool = num_blocks * w.num_kv_heads * w.block_size * w.head_dim * 2 * 2
    return int(min(16, max(1, -(-REPLICA_TARGET_BYTES // pool))))


class Scenario:
    """Resident state of one benchmark: cache, requests and per-step device inputs."""

    def __init__(self, w, cache, seqs, lengths, step_k, step_v, step_q, max_blocks, out,
                 unique_bytes=None, extra=None):
        self.w, self.cache, self.seqs, self.lengths = w, cache, seqs, lengths
        self.step_k, self.step_v, self.step_q = step_k, step_v, step_q
        self.max_blocks, self.out = max_blocks, out
        self.unique_bytes = unique_bytes
        self.extra = extra or {}

    @property
    def num_seqs(self):
        return len(self.seqs)

    def workspace(self, part, max_len):
        return self.cache.workspace(self.num_seqs, self.w.num_q_heads, max_len, part)

    def step(self, t, partition, timer, plans, marks=None):
        cache = self.cache
        layer = t % len(cache.k)            # the pool replica this step writes and reads
        # reserve, tables, plan and the new tokens' write: one host call, one launch
        _, batch = cache.decode_step(self.seqs, self.max_blocks, partition_size=partition,
                                     k_new=self.step_k[t], v_new=self.step_v[t], layer=layer,
                                     marks=marks)
        grouped = batch.group_items_dev is not None
        plans.append(dict(batch.plan,
                          num_groups=batch.groups_dev.shape[0] if grouped else 0,
                          num_group_items=batch.group_items_dev.shape[0] if grouped else 0))
        cache.attend(self.step_q[t], batch, self.w.scale, layer=layer, out=self.out,
                     timing=timer)


def _to_dev(arrays, dev):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrays]


def decode_scenario(w, total_steps, dev, replicas=0):
    """Requests whose first L-1 tokens are cached; step t appends one token to each.
    The pool exists in ``replicas`` copies with identical contents and tables."""
    import torch

    from paged_kv_cache_244_amd import workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    # Room for the tokens appended during the run: one more block per request per B steps.
    growth = w.num_seqs * (-(-total_steps // w.block_size) + 1)
    num_blocks = w.num_blocks + growth
    order = np.concatenate([w.initial_order, np.arange(w.num_blocks, num_blocks, dtype=np.int32)])
    nrep = replicas_for(num_blocks, w, replicas)
    cache = PagedKVCache(num_blocks, w.num_kv_heads, w.head_dim, w.block_size, num_layers=nrep,
                         initial_order=order, device=dev, poison=False, num_q_heads=w.num_q_heads,
                         q_dtype=torch.float16 if w.q.dtype == np.float16 else torch.float32)
    seqs = [cache.new_sequence() for _ in range(w.num_seqs)]
    prompt_idx = np.concatenate([np.arange(o, o + L - 1) for o, L in zip(w.offsets[:-1], w.lengths)])
    slots = cache.reserve_many(seqs, [int(L) - 1 for L in w.lengths])
    pk, pv = _to_dev([w.k_tokens[prompt_idx], w.v_tokens[prompt_idx]], dev)
    for layer in range(nrep):
        cache.write(slots, pk, pv, layer=layer)
    del pk, pv
    last_idx = w.offsets[:-1] + w.lengths - 1
    step_k, step_v, step_q = [], [], []
    for t in range(total_steps):
        k, v, q = ((w.k_tokens[last_idx], w.v_tokens[last_idx], w.q) if t == 0
                   else workloads.step_inputs(w, t))
        dk, dv, dq = _to_dev([k, v, q], dev)
        step_k.append(dk)
        step_v.append(dv)
        step_q.append(dq)
    max_blocks = -(-(int(w.lengths.max()) + total_steps) // w.block_size)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    return Scenario(w, cache, seqs, w.lengths.astype(np.int64) - 1, step_k, step_v, step_q,
                    max_blocks, out, extra={"pool_replicas": nrep})


def sampling_scenario(sw, total_steps, dev, replicas=0, prefix_groups=True):
    """Prompts forked into samples sharing their blocks; the first step copies the
    partly filled last prompt block of every sample but one per prompt."""
    import torch

    from paged_kv_cache_244_amd.cache import PagedKVCache

    if total_steps > sw.steps:
        raise SystemExit(f"parallel_sampling has {sw.steps} steps; asked for {total_steps}")
    nrep = replicas_for(sw.num_blocks, sw, replicas)
    cache = PagedKVCache(sw.num_blocks, sw.num_kv_heads, sw.head_dim, sw.block_size,
                         num_layers=nrep, initial_order=sw.initial_order, device=dev, poison=False,
                         num_q_heads=sw.num_q_heads, prefix_groups=prefix_groups)
    prompts = [cache.new_sequence() for _ in range(sw.num_prompts)]
    slots = cache.reserve_many(prompts, sw.prompt_lengths)
    pk, pv = _to_dev([sw.prompt_k, sw.prompt_v], dev)
    for layer in range(nrep):
        cache.write(slots, pk, pv, layer=layer)
    del pk, pv
    seqs = []
    for p in prompts:
        seqs.extend(cache.fork(p) for _ in range(sw.samples))
        cache.free(p)
    step_k, step_v, step_q = [], [], []
    for t in range(total_steps):
        dk, dv, dq = _to_dev(list(sw.step_inputs(t)), dev)
        step_k.append(dk)
        step_v.append(dv)
        step_q.append(dq)
    lengths = np.repeat(sw.prompt_lengths.astype(np.int64), sw.samples)
    max_blocks = -(-(int(lengths.max()) + total_steps) // sw.block_size)
    out = torch.empty((len(seqs), sw.num_q_heads, sw.head_dim), dtype=torch.float32, device=dev)
    tok_bytes = 2 * sw.num_kv_heads * sw.head_dim * 2
    B = sw.block_size

    def unique_bytes(lens):
        # Shared full prompt blocks are stored (and read from HBM) once per prompt.
        shared = sum(int(P) // B * B for P in sw.prompt_lengths)
        own = int(np.sum(lens)) - sw.samples * shared
        return (shared + own) * tok_bytes

    w = SimpleWorkload(sw.name, sw.num_q_heads, sw.num_kv_heads, sw.head_dim, sw.block_size,
                       np.float16, sw.scale)
    return Scenario(w, cache, seqs, lengths, step_k, step_v, step_q, max_blocks, out,
                    unique_bytes=unique_bytes,
                    extra={"pool_replicas": nrep,
                           "prompts": sw.num_prompts, "samples_per_prompt": sw.samples,
                           "note": "value counts logical K/V bytes; shared prompt blocks are "
                                   "read by every sample"})


class ContiguousScenario:
    """The same requests, data and per-step inputs in the layout without a block
    table: K and V rows [S, Hkv, Lmax, D] per replica.  The new token of each step
    is stored with a torch index (plumbing of this comparison layout, outside the
    timed decode launch); the launch schedule comes from the same planner."""

    def __init__(self, base, total_steps, dev, replicas):
        import torch

        from paged_kv_cache_244_amd.cache import _Staging

        w = base.w
        self.w, self.seqs, self.lengths = w, base.seqs, base.lengths
        self.step_k, self.step_v, self.step_q, self.out = base.step_k, base.step_v, base.step_q, base.out
        self.unique_bytes, self.extra = None, {}
        S, hkv, d = len(base.seqs), w.num_kv_heads, w.head_dim
        self.lmax = -(-(int(base.lengths.max()) + total_steps) // 16) * 16
        row_bytes = S * hkv * self.lmax * d * 2 * 2
        nrep = replicas if replicas > 0 else int(min(16, max(1, -(-REPLICA_TARGET_BYTES // row_bytes))))
        self.k = [torch.zeros((S, hkv, self.lmax, d), dtype=torch.float16, device=dev)
                  for _ in range(nrep)]
        self.v = [torch.zeros_like(self.k[0]) for _ in range(nrep)]
        # Prompt tokens: request i's first L_i - 1 tokens, in logical order.
        lens0 = base.lengths.astype(np.int64)
        seq_idx = np.repeat(np.arange(S), lens0)
        pos_idx = np.concatenate([np.arange(L) for L in lens0]) if S else np.zeros(0, np.int64)
        tok_idx = np.concatenate([np.arange(o, o + L) for o, L in zip(w.offsets[:-1], lens0)])
        si, pi = (torch.from_numpy(a).to(dev) for a in (seq_idx, pos_idx))
        kt, vt = _to_dev([w.k_tokens[tok_idx], w.v_tokens[tok_idx]], dev)
        for r in range(nrep):
            self.k[r][si, :, pi, :] = kt
            self.v[r][si, :, pi, :] = vt
        del kt, vt
        self.lens = lens0.astype(np.int32)          # cached tokens per request
        self.staging = _Staging(dev)
        self.arange = torch.arange(S, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.ws = None
        self.extra = {"pool_replicas": nrep, "layout": "contiguous", "row_tokens": self.lmax}

    @property
    def num_seqs(self):
        return len(self.seqs)

    def workspace(self, part, max_len):
        import torch
        need = _lib_mod().pa_decode_workspace_size(self.num_seqs, self.w.num_q_heads,
                                                   self.w.head_dim, max_len, part)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.out.device)
        return self.ws if need else None

    def step(self, t, partition, timer, plans, marks=None):
        _lib = _lib_mod()
        w, r = self.w, t % len(self.k)
        pos = self.lens.copy()
        self.lens += 1
        qd = _lib.PKV_F16 if self.step_q[t].dtype.itemsize == 2 else _lib.PKV_F32
        items, plan = _lib.plan(self.lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 16, qd,
                                partition_size=partition)
        plans.append(plan)
        lens_d, pos_d, items_d = self.staging.upload([self.lens, pos.astype(np.int64),
                                                      items.view(np.int32)], self.stream)
        self.k[r][self.arange, :, pos_d, :] = self.step_k[t]
        self.v[r][self.arange, :, pos_d, :] = self.step_v[t]
        max_len = int(self.lens.max())
        ws = self.workspace(plan["partition_size"], max_len)
        if timer is not None:
            _lib.time_next_call(timer)
        _lib.pa_decode_contiguous(self.out, self.step_q[t], self.k[r], self.v[r], lens_d, w.scale,
                                  max_len, partition_size=plan["partition_size"], workspace=ws,
                                  stream=self.stream, work_items=items_d,
                                  waves_per_cu=plan["waves_per_cu"])


def _lib_mod():
    from paged_kv_cache_244_amd import _lib
    return _lib


class SimpleWorkload:
    def __init__(self, name, hq, hkv, d, b, q_dtype, scale):
        self.name, self.num_q_heads, self.num_kv_heads = name, hq, hkv
        self.head_dim, self.block_size, self.q_dtype, self.scale = d, b, q_dtype, scale


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak


def prefill_bench(args):
    """Prompt phase: each step admits the 16 prompts (host allocator, one upload), writes
    their K/V, runs pa_prefill over the block tables, then frees them.  Metric: causal
    attention FLOP/s (roofline: the fp16 matrix cores)."""
    import torch

    from paged_kv_cache_244_amd import workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    dev = torch.device("cuda:0")
    w = workloads.prefill()
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                         initial_order=w.initial_order, device=dev, poison=False,
                         num_q_heads=w.num_q_heads)
    kd, vd, qd = _to_dev([w.k_tokens, w.v_tokens, w.q], dev)
    out = torch.empty(qd.shape, dtype=torch.float32, device=dev)
    lens = [int(L) for L in w.lengths]
    stream = cache.stream
    ring = timer_ring()

    def step(slot=None):
        seqs = [cache.new_sequence() for _ in lens]
        slots = cache.reserve_many(seqs, lens)
        cache.write(slots, kd, vd)
        cache.prefill(qd, seqs, lens, w.scale, out=out,
                      timing=ring.take(slot) if slot is not None else None)
        for sq in seqs:
            cache.free(sq)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    every = max(1, args.time_every)
    for i in range(args.steps):
        step(i if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = list(ring.results().values())
    flops = float(w.flops())
    achieved = flops / (float(np.mean(ms)) / 1e3) / 1e12
    baseline = None
    if args.cpu_seconds > 0:
        baseline = prefill_cpu_baseline(w)
    counters = counter_traffic(None, kernel="pa_prefill")
    result = {
        "metric": "paged prefill attention TFLOP/s (% of fp16 matrix peak)",
        "value": round(flops * args.steps / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "prefill: 16 prompts of U{512..4096} tokens", "num_seqs": w.num_seqs,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "prompt_tokens": int(w.lengths.sum()),
                   "flops_per_step": int(flops)},
        "prefill_us": round(float(np.mean(ms)) * 1e3, 2),
        "prefill_timing": f"kernel-level HIP events on every {every}th timed step",
        "prefill_us_p10_p90": [round(float(np.percentile(ms, 10)) * 1e3, 2),
                               round(float(np.percentile(ms, 90)) * 1e3, 2)],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": counters["traffic_bytes_per_launch"] if counters else None,
                     "kernel": "pa_prefill"},
        "cpu_baseline": baseline,
        "gpu": GPU_INFO,
    }
    print(json.dumps(result), flush=True)


PCIE_PEAK_GBS = 63.0   # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def swap_bench(args):
    """Eviction to the host tier: each step swaps every other request of the OPT-13B
    decode batch out to pinned host memory and back in (the allocator picks the
    blocks, one upload of the pairs, kv_swap_blocks per direction on one stream).
    Metric: K/V bytes moved per second; roofline: the copy kernel against one
    direction of the host link.  The runtime's own copy (hipMemcpyAsync through
    torch) of one contiguous buffer of the same size, each way, is reported
    beside it as the rate of the link without block gathering."""
    import torch

    from paged_kv_cache_244_amd import workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    dev = torch.device("cuda:0")
    w = workloads.opt13b()
    lens = [int(L) for L in w.lengths]
    bs = w.block_size
    block_bytes = 2 * w.num_kv_heads * bs * w.head_dim * 2          # K and V of one block
    moved_idx = list(range(0, len(lens), 2))
    moved_blocks = sum(-(-lens[i] // bs) for i in moved_idx)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, bs,
                         initial_order=w.initial_order, device=dev, poison=False,
                         num_q_heads=w.num_q_heads, host_blocks=moved_blocks)
    kd, vd = _to_dev([w.k_tokens, w.v_tokens], dev)
    seqs = [cache.new_sequence() for _ in lens]
    cache.write(cache.reserve_many(seqs, lens), kd, vd)
    moved = [seqs[i] for i in moved_idx]
    def read(e):
        e[3].synchronize()
        return e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])

    ring = TimingRing(4, lambda: [torch.cuda.Event(enable_timing=True) for _ in range(4)], read)

    def step(slot=None):
        e = ring.take(slot) if slot is not None else None
        n_out = cache.swap_out(moved, events=None if e is None else (e[0], e[1]))
        n_in = cache.swap_in(moved, events=None if e is None else (e[2], e[3]))
        assert n_out == n_in == moved_blocks

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = list(ring.results().values())
    out_ms = [t[0] for t in times]
    in_ms = [t[1] for t in times]
    nbytes = moved_blocks * block_bytes
    gbs = lambda ms: nbytes / (ms / 1e3) / 1e9  # noqa: E731
    achieved = gbs(float(np.mean(out_ms + in_ms)))
    runtime_copy = runtime_copy_rates(nbytes, dev)
    baseline = swap_cpu_baseline(w) if args.cpu_seconds > 0 else None
    result = {
        "metric": "swap to host tier: K/V GB/s moved (% of one direction of PCIe 5.0 x16)",
        "value": round(2 * nbytes * args.steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "swap: every other request of the OPT-13B decode batch out and in",
                   "requests_moved": len(moved), "blocks_moved": moved_blocks,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": bs,
                   "bytes_per_direction": nbytes},
        "swap_out_us": round(float(np.mean(out_ms)) * 1e3, 1),
        "swap_in_us": round(float(np.mean(in_ms)) * 1e3, 1),
        "swap_out_gbs": round(gbs(float(np.mean(out_ms))), 2),
        "swap_in_gbs": round(gbs(float(np.mean(in_ms))), 2),
        "runtime_copy_gbs": runtime_copy,
        "roofline": {"bound": "pcie", "achieved": round(achieved, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "kv_copy_blocks_kernel (kv_swap_blocks)"},
        "cpu_baseline": baseline,
        "gpu": GPU_INFO,
    }
    print(json.dumps(result), flush=True)


def runtime_copy_rates(nbytes, dev, reps=5):
    """One contiguous device <-> pinned host transfer of ``nbytes`` through the runtime's
    copy path (torch copy_ -> hipMemcpyAsync; the runtime picks a blit kernel or a copy
    engine), each direction: the link's rate without block gathering."""
    import torch

    d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    rates = {}
    for name, dst, src in (("d2h", h, d), ("h2d", d, h)):
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        rates[name] = round(nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9, 2)
    return rates


def swap_cpu_baseline(w, blocks=512):
    """The oracle's copy_blocks_between moving ``blocks`` blocks between two host pools."""
    from oracle import cache

    shape = (blocks, w.num_kv_heads, w.block_size, w.head_dim)
    src = [(np.ones(shape, np.float16), np.ones(shape, np.float16))]
    dst = [(np.zeros(shape, np.float16), np.zeros(shape, np.float16))]
    pairs = np.stack([np.arange(blocks), np.random.default_rng(0).permutation(blocks)], 1)
    t0 = time.perf_counter()
    cache.copy_blocks_between(src, dst, pairs)
    dt = time.perf_counter() - t0
    nbytes = blocks * 2 * int(np.prod(shape[1:])) * 2
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{blocks} OPT-13B blocks (K and V) between two host pools, numpy",
            "seconds": round(dt, 3)}


def _beam_replay(w, steps):
    """The churn schedule on a host-only allocator (same initial order, same calls as
    the cache makes): per step the logical and unique (distinct blocks' filled slots)
    tokens attention reads, and the copy-on-write pairs of the step's append."""
    _lib = _lib_mod()
    a = _lib.BlockAllocator(w.num_blocks, w.block_size, w.initial_order)
    groups = []
    for L in w.prompt_lengths:
        s = a.create()
        a.append(s, int(L))
        groups.append([s] + [a.fork(s) for _ in range(w.beams - 1)])
    logical, unique, pairs = [], [], []
    bs = w.block_size
    for t in range(steps):
        groups = _beam_prune(w, t, groups, a.free, a.fork)
        seqs = [s for g in groups for s in g]
        _, p = a.append_batch(seqs)
        pairs.append(int(p.shape[0]))
        lens = a.lengths(seqs)
        tables, _ = a.export(seqs, int(max(lens) + bs - 1) // bs, -1)
        fill = {}
        for row, L in zip(tables, lens):
            for j in range(-(-int(L) // bs)):
                fill[int(row[j])] = min(bs, int(L) - j * bs)
        logical.append(int(lens.sum()))
        unique.append(sum(fill.values()))
    return logical, unique, pairs


def _beam_prune(w, t, groups, free, fork, plan=False):
    """Cancel and fork beams per the workload's schedule for step t (``plan``: that
    schedule, drawn beforehand, or False to draw it here)."""
    if plan is False:
        plan = w.prune_plan(t)
    if plan is None:
        return groups
    out = []
    for g, (drop, src) in zip(groups, plan):
        for i in drop:
            free(g[i])
        keep = [s for i, s in enumerate(g) if i not in drop]
        out.append(keep + [fork(g[j]) for j in src])
    return out


def churn_bench(args):
    """Beam-search-like churn: 8 prompts x 8 beams (OPT-13B attention shape); every
    step appends one token to each of the 64 beams and attends; every 4th step each
    prompt cancels 4 beams and forks 4 survivors, so copy-on-write copies (every
    layer) and immediate reuse of freed blocks recur with work queued.  The pool has
    several layers (>= 2 GiB, one written and read per step, as a model's layers
    would be); copies go to every layer.  Metric: generated tokens per second;
    roofline: decode attention over the unique K/V bytes it reads."""
    import torch

    from paged_kv_cache_244_amd import workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    dev = torch.device("cuda:0")
    w = workloads.beams()
    total_steps = args.warmup + args.steps
    tok_bytes = 2 * w.num_kv_heads * w.head_dim * 2
    layers = max(1, -(-(2 << 30) // (w.num_blocks * w.block_size * tok_bytes)))
    logical, unique, pairs = _beam_replay(w, total_steps)
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                         num_layers=layers, initial_order=w.initial_order, device=dev, poison=False,
                         num_q_heads=w.num_q_heads, prefix_groups=not args.no_prefix_groups)
    pk, pv = _to_dev([w.prompt_k, w.prompt_v], dev)
    groups = []
    for L in w.prompt_lengths:
        s = cache.new_sequence()
        groups.append([s])
    slots = cache.reserve_many([g[0] for g in groups], [int(L) for L in w.prompt_lengths])
    for layer in range(layers):
        cache.write(slots, pk, pv, layer=layer)
    for g in groups:
        g.extend(cache.fork(g[0]) for _ in range(w.beams - 1))
    inputs = [_to_dev(list(w.step_inputs(t)), dev) for t in range(total_steps)]
    out = torch.empty((w.num_prompts * w.beams, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device=dev)
    ring = timer_ring()

    part = "auto" if args.partition == "auto" else int(args.partition)
    # The cancel/fork schedule is the workload's input: drawn before timing, so the
    # timed steps hold the allocator's forks and frees but not the random draws.
    schedule = [w.prune_plan(t) for t in range(total_steps)]

    def step(t, e=None):
        nonlocal groups
        groups = _beam_prune(w, t, groups, cache.free, cache.fork, schedule[t])
        seqs = [s for g in groups for s in g]
        k, v, q = inputs[t]
        layer = t % layers
        _, batch = cache.decode_step(seqs, k_new=k, v_new=v, layer=layer, partition_size=part)
        cache.attend(q, batch, w.scale, layer=layer, out=out, timing=e)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    every = max(1, args.time_every)
    for i in range(args.steps):
        step(args.warmup + i, ring.take(i) if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    by_step = ring.results()
    sampled = sorted(by_step)
    ms = [by_step[i] for i in sampled]
    timed = slice(args.warmup, total_steps)
    # The roofline: unique bytes of the steps whose decode was timed over their mean time.
    uniq = float(np.mean([unique[args.warmup + i] for i in sampled])) * tok_bytes
    uniq_all = float(np.mean(unique[timed])) * tok_bytes
    logi = float(np.mean(logical[timed])) * tok_bytes
    dec_s = float(np.mean(ms)) / 1e3
    achieved = uniq / dec_s / 1e9
    s_count = w.num_prompts * w.beams
    result = {
        "metric": "beam-search churn: generated tokens/s (decode roofline on unique K/V bytes)",
        "value": round(s_count * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "beams: 8 prompts of U{256..1024} tokens x 8 beams, prune 4 and fork 4 "
                               "every 4 steps", "requests": s_count, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "layers": layers, "cow_pairs_per_step": round(float(np.mean(pairs[timed])), 2),
                   "prefix_groups": not args.no_prefix_groups,
                   "unique_kv_bytes_per_step": int(uniq_all), "logical_kv_bytes_per_step": int(logi)},
        "decode_us": round(dec_s * 1e6, 2),
        "decode_timing": f"kernel-level HIP events on every {every}th timed step",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_decode"},
        "cpu_baseline": None,
        "gpu": GPU_INFO,
    }
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(w, prompt=1024):
    """The oracle's attend_prefill_paged on one request's first ``prompt`` tokens."""
    from threadpoolctl import threadpool_limits

    from oracle import attention, cache

    nb = -(-prompt // w.block_size)
    shape = (nb, w.num_kv_heads, w.block_size, w.head_dim)
    kp, vp = np.zeros(shape, np.float16), np.zeros(shape, np.float16)
    cache.write_slots(kp, vp, w.k_tokens[:prompt], w.v_tokens[:prompt], list(range(prompt)),
                      w.block_size)
    tables = np.arange(nb, dtype=np.int64)[None]
    starts = np.array([0, prompt], dtype=np.int64)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        attention.attend_prefill_paged(w.q[:prompt], kp, vp, tables, [prompt], starts,
                                       w.block_size, w.scale)
        dt = time.perf_counter() - t0
    flops = 4 * w.num_q_heads * w.head_dim * prompt * (prompt + 1) // 2
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"one prompt of {prompt} tokens, fp64 numpy attend_prefill_paged",
            "seconds": round(dt, 2)}


def write_copy_times(marks, sc, w):
    """Kernel times of the step's other launches, from the events decode_step
    passed to the library: the upload of the step buffer fused with the new
    tokens' write (steps without copies), or on copy-on-write steps the upload,
    the block copy (every pool replica) and the separate write.  Bytes are algorithmic: a write moves
    T tokens of K and V in and out; a copy reads and writes whole blocks."""
    tok = 2 * w.num_kv_heads * w.head_dim * 2                     # K+V bytes of one token
    block = tok * w.block_size
    layers = len(sc.cache.k)
    t = sc.num_seqs
    fused, upload, copy, write, pairs = [], [], [], [], []
    for m in marks:                      # (pairs, upload ms[, copy ms, write ms]) per step
        if m[0]:
            pairs.append(m[0])
            upload.append(m[1])
            copy.append(m[2])
            write.append(m[3])
        else:
            fused.append(m[1])

    def rate(nbytes, ms):
        gbs = nbytes / (ms / 1e3) / 1e9
        return round(gbs, 1), round(gbs / HBM_PEAK_GBS, 4)

    res = {"write_bytes_per_step": 2 * t * tok}
    if fused:
        res["upload_write_us"] = round(float(np.mean(fused)) * 1e3, 2)
        res["upload_write_steps"] = len(fused)
    if copy:
        cbytes = 2 * float(np.mean(pairs)) * layers * block
        cms = float(np.mean(copy))
        wms = float(np.mean(write))
        res.update({
            "copy_steps": len(copy), "copy_pairs_per_step": round(float(np.mean(pairs)), 1),
            "copy_layers": layers, "copy_bytes_per_step": int(cbytes),
            "copy_us": round(cms * 1e3, 2), "copy_gbs_frac": rate(cbytes, cms),
            "write_us": round(wms * 1e3, 2), "write_gbs_frac": rate(2 * t * tok, wms),
            "upload_us_copy_steps": round(float(np.mean(upload)) * 1e3, 2)})
    return res


def summarize_timeline(recs, w):
    """Text summary of per-wave timeline records (pkv_wave_timeline_read layout)."""
    recs = recs[recs[:, 0] > 0]
    if len(recs) == 0:
        return "no waves recorded"
    rt0, rt1 = recs[:, 0].astype(np.int64), recs[:, 1].astype(np.int64)
    t0 = rt0.min()
    st, en = (rt0 - t0) / 100.0, (rt1 - t0) / 100.0          # 100 MHz real-time counter
    dur = np.maximum(en - st, 1e-3)
    c1 = (recs[:, 2] & 0xFFFFFFFF).astype(float)
    c2 = (recs[:, 2] >> 32).astype(float)
    c3 = (recs[:, 3] & 0xFFFFFFFF).astype(float)
    c4 = (recs[:, 3] >> 32).astype(float)
    xcc = (recs[:, 4] & 0xFFFFFFFF).astype(np.int64) % 8
    tiles = (recs[:, 4] >> 32).astype(np.int64)
    tokens = (recs[:, 5] >> 40).astype(np.int64)
    clk = float(np.median(c4 / dur))                        # shader-clock ticks per us
    span = float(en.max())
    kv_bytes_tok = 2 * w.head_dim * 2                       # K and V of one token, one KV head
    nbytes = float(np.sum(tokens)) * kv_bytes_tok
    lines = [f"waves {len(recs)}, launch span {span:.1f} us (first start to last end), "
             f"{nbytes / 1e6:.1f} MB of K/V streamed ({nbytes / span / 1e6:.2f} TB/s over the span), "
             f"shader clock ~{clk / 1e3:.2f} GHz",
             f"start-up, mean (median) us: work-list entry {np.mean(c1) / clk:.2f} ({np.median(c1) / clk:.2f}), "
             f"then table row, query and length {np.mean(c2 - c1) / clk:.2f} ({np.median(c2 - c1) / clk:.2f}), "
             f"then first tile {np.mean(c3 - c2) / clk:.2f} ({np.median(c3 - c2) / clk:.2f})",
             f"tiles per wave p10/p50/p90/max: {np.percentile(tiles, [10, 50, 90, 100]).astype(int).tolist()}; "
             f"wave time p10/p50/p90 {np.round(np.percentile(dur, [10, 50, 90]), 1).tolist()} us",
             "by start time (5 us bins): waves, then mean us to entry / inputs / first tile, and us per "
             "further tile of waves with >= 8 tiles:"]
    for lo in range(0, int(st.max()) + 5, 5):
        m = (st >= lo) & (st < lo + 5)
        if not m.any():
            continue
        mm = m & (tiles >= 8)
        per = (float(np.mean((c4[mm] - c3[mm]) / clk / (tiles[mm] - 1))) if mm.any() else float("nan"))
        lines.append(f"  {lo:4d}-{lo + 5:<4d} {int(m.sum()):5d}  {np.mean(c1[m]) / clk:5.2f} "
                     f"{np.mean(c2[m] - c1[m]) / clk:5.2f} {np.mean(c3[m] - c2[m]) / clk:5.2f}  {per:5.2f}")
    grid = np.arange(0.0, span + 2.0, 2.0)
    lines.append("resident waves every 2 us: " + " ".join(str(int(((st <= g) & (en > g)).sum())) for g in grid))
    lines.append("by XCD: waves, wave time (ms), MB streamed, us per tile of waves with >= 8 tiles, last end (us):")
    for x in range(8):
        m = xcc == x
        if not m.any():
            continue
        mm = m & (tiles >= 8)
        per = float(np.mean((c4[mm] - c3[mm]) / clk / (tiles[mm] - 1))) if mm.any() else float("nan")
        lines.append(f"  XCD {x}: {int(m.sum()):5d} {float(np.sum(dur[m])) / 1e3:7.2f} "
                     f"{float(np.sum(tokens[m])) * kv_bytes_tok / 1e6:7.1f} {per:5.2f} {float(en[m].max()):7.1f}")
    return "\n".join(lines)


PAIR_STRETCHES = ("from the last pair (its end barrier)", "first-half load issue", "first-half work",
                  "between the halves", "second-half load issue", "second-half work", "load wait")


def prefill_timeline(args, dev):
    """--timeline for prefill: args.warmup prefill steps, then one recorded launch;
    prints each wave's mean shader-clock cycles per tile pair by stretch."""
    import torch

    from paged_kv_cache_244_amd import _lib, workloads
    from paged_kv_cache_244_amd.cache import PagedKVCache

    w = workloads.prefill()
    cache = PagedKVCache(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                         initial_order=w.initial_order, device=dev, poison=False,
                         num_q_heads=w.num_q_heads)
    kd, vd, qd = _to_dev([w.k_tokens, w.v_tokens, w.q], dev)
    out = torch.empty(qd.shape, dtype=torch.float32, device=dev)
    lens = [int(L) for L in w.lengths]

    def step():
        seqs = [cache.new_sequence() for _ in lens]
        cache.write(cache.reserve_many(seqs, lens), kd, vd)
        cache.prefill(qd, seqs, lens, w.scale, out=out)
        for sq in seqs:
            cache.free(sq)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.wave_timeline_read(_lib.PKV_TIMELINE_PREFILL, clear=True)
    step()
    torch.cuda.synchronize()
    recs = _lib.wave_timeline_read(_lib.PKV_TIMELINE_PREFILL)
    recs = recs[(recs[:, 3] >> 32) > 0]                      # waves that summed some pairs
    print(f"tile-pair timeline: workload prefill, launch after {args.warmup} warmup steps; "
          f"{len(recs)} waves of {len(recs) // 8} full workgroups of head tile 0 with tile pairs 8-39")
    if len(recs) == 0:
        return
    halves = np.stack([recs[:, 0] & 0xFFFFFFFF, recs[:, 0] >> 32, recs[:, 1] & 0xFFFFFFFF,
                       recs[:, 1] >> 32, recs[:, 2] & 0xFFFFFFFF, recs[:, 2] >> 32,
                       recs[:, 3] & 0xFFFFFFFF], axis=1).astype(float)
    per_pair = halves / (recs[:, 3] >> 32).astype(float)[:, None]
    wave = (recs[:, 4] >> 32).astype(int)
    print("mean shader-clock cycles per tile pair, by wave (waves 0-3: matrix phase first; "
          "4-7: softmax and K loads first):")
    print("  wave  " + " | ".join(PAIR_STRETCHES) + " | pair")
    for wv in range(8):
        m = wave == wv
        if m.any():
            v = per_pair[m].mean(axis=0)
            print(f"  {wv}     " + "  ".join(f"{x:6.0f}" for x in v) + f"  {v.sum():6.0f}")
    print(f"pair: {per_pair.sum(axis=1).mean():.0f} cycles on average over the recorded waves", flush=True)


def wave_timeline(args):
    """--timeline: the per-wave timeline of one decode launch, recorded by the
    instrumented library after args.warmup steps; prints a text summary."""
    import torch

    from paged_kv_cache_244_amd import _lib, workloads

    if args.workload not in ("opt13b", "gqa", "long_context", "tiny", "prefill"):
        raise SystemExit("--timeline records the decode workloads opt13b, gqa, long_context, "
                         "tiny and the prefill workload")
    if not os.path.exists(_lib.TIMELINE_LIB_PATH):
        raise SystemExit(f"{_lib.TIMELINE_LIB_PATH} is missing: "
                         "python -m paged_kv_cache_244_amd.build --timeline")
    _lib.LIB_PATH = _lib.TIMELINE_LIB_PATH                 # before the library is first loaded
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "prefill":
        prefill_timeline(args, dev)
        return
    _lib.set_kernel_policy(_lib.PKV_POLICY_VALU if args.kernel_policy == "valu"
                           else _lib.PKV_POLICY_DEFAULT)
    w = {"long_context": lambda: workloads.long_context(16),
         "tiny": workloads.tiny}.get(args.workload, workloads.WORKLOADS.get(args.workload))()
    total = args.warmup + 1
    sc = decode_scenario(w, total, dev, args.replicas)
    qd = _lib.PKV_F16 if w.q_dtype == np.float16 else _lib.PKV_F32
    partition = (_lib.plan(sc.lengths + total, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.block_size, qd)[1]["partition_size"]
                 if args.partition == "auto" else int(args.partition))
    sc.workspace(partition, int(sc.lengths.max()) + total)
    plans = []
    for t in range(args.warmup):
        sc.step(t, partition, None, plans)
    torch.cuda.synchronize()
    kinds = (_lib.PKV_TIMELINE_VALU, _lib.PKV_TIMELINE_MFMA)
    for k in kinds:
        _lib.wave_timeline_read(k, clear=True)
    sc.step(args.warmup, partition, None, plans)
    torch.cuda.synchronize()
    recs = np.concatenate([_lib.wave_timeline_read(k) for k in kinds])
    plan = {k: v for k, v in plans[-1].items() if not hasattr(v, "__len__")}
    print(f"per-wave timeline: workload {args.workload}, step {args.warmup} after {args.warmup} "
          f"warmup steps, plan {plan}")
    print(summarize_timeline(recs, w), flush=True)


def main():
    args = parse_args()
    if args.timeline:
        wave_timeline(args)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.stream_probe:
        stream_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path has no multi-GPU sharding in this build)", file=sys.stderr)
        sys.exit(2)
    global GPU_INFO
    GPU_INFO = gpu_info()                   # before this process touches the GPU
    if args.workload in ("prefill", "swap", "beams"):
        if args.steps is None:
            args.steps = 50
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        torch.cuda.set_device(0)
        {"prefill": prefill_bench, "swap": swap_bench, "beams": churn_bench}[args.workload](args)
        return

    import torch

    from paged_kv_cache_244_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    from paged_kv_cache_244_amd import _lib
    _lib.set_kernel_policy(_lib.PKV_POLICY_VALU if args.kernel_policy == "valu"
                           else _lib.PKV_POLICY_DEFAULT)

    ps = args.workload == "parallel_sampling"
    if ps:
        # The workload's statement: 128 steps from the fork on, step 0 being the one
        # that copies the partly filled last prompt block.  The timed run starts
        # at step 0 on a fresh cache; the warmup runs on a separate one.
        sw = workloads.parallel_sampling()
        if args.steps is None:
            args.steps = sw.steps
        if args.warmup:
            warm = sampling_scenario(sw, args.warmup, dev, args.replicas,
                                     prefix_groups=not args.no_prefix_groups)
            for t in range(args.warmup):
                warm.step(t, "auto", None, [])
            torch.cuda.synchronize()
            del warm
            torch.cuda.empty_cache()
        first_step = 0
        sc = sampling_scenario(sw, args.steps, dev, args.replicas,
                               prefix_groups=not args.no_prefix_groups)
    else:
        if args.steps is None:
            args.steps = 50
        first_step = args.warmup
        w = {"long_context": lambda: workloads.long_context(16),
             "tiny": workloads.tiny}.get(args.workload, workloads.WORKLOADS.get(args.workload))()
        if args.block_size and args.block_size != w.block_size:
            w = workloads.with_block_size(w, args.block_size)
        sc = decode_scenario(w, args.warmup + args.steps, dev, args.replicas)
        if args.layout == "contiguous":
            base = sc
            sc = ContiguousScenario(base, args.warmup + args.steps, dev, args.replicas)
            del base
            torch.cuda.empty_cache()
    if args.layout == "contiguous" and ps:
        raise SystemExit("the contiguous layout is measured on the decode workloads only")
    if ps and args.block_size and args.block_size != 16:
        raise SystemExit("--block-size applies to the decode workloads, not parallel_sampling")
    total_steps = first_step + args.steps
    w = sc.w
    # The planner's automatic choice for the lengths the run ends at (they grow by
    # total_steps tokens), then kept fixed so every timed step runs one schedule shape.
    qd = _lib.PKV_F16 if w.q_dtype == np.float16 else _lib.PKV_F32
    partition = (_lib.plan(sc.lengths + total_steps, w.num_q_heads, w.num_kv_heads, w.head_dim,
                           w.block_size, qd)[1]["partition_size"]
                 if args.partition == "auto" else int(args.partition))
    sc.workspace(partition, int(sc.lengths.max()) + total_steps)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    every = max(1, args.time_every)
    # Decode: marker events on every `every`-th timed step.  Other launches of the
    # step (upload and write, copy-on-write copies): the kernels' own start and end
    # (kernel-level events) on every 2*every-th step, shifted, and on the first step
    # of a parallel-sampling run, whose copies follow a synchronisation.
    decode_ring = timer_ring(4)
    mark_steps = {i for i in range(args.steps) if i % (2 * every) == every // 2 + every}
    if ps:
        mark_steps.add(0)

    def read_marks(m):
        if m["pairs"]:
            return (m["pairs"], m["upload"].ms(), m["copy"].ms(), m["write"].ms())
        return (0, m["upload"].ms())

    mark_ring = TimingRing(4, lambda: dict(zip(("upload", "copy", "write"), kernel_timers(3))),
                           read_marks)
    torch.cuda.synchronize()
    step_bytes, unique_step_bytes = [], []
    plans = []

    lengths = sc.lengths.copy()
    for t in range(first_step):
        sc.step(t, partition, None, plans)
        lengths += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev = decode_ring.take(i) if i % every == 0 else None
        marks = mark_ring.take(i) if args.layout == "paged" and i in mark_steps else None
        sc.step(first_step + i, partition, ev, plans, marks)
        lengths += 1
        step_bytes.append(kv_bytes(lengths, w))
        if sc.unique_bytes is not None:
            unique_step_bytes.append(sc.unique_bytes(lengths))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    decode_by_step = decode_ring.results()
    timed = sorted(decode_by_step)
    decode_ms = [decode_by_step[i] for i in timed]
    decode_avg_s = float(np.mean(decode_ms)) / 1e3
    total_bytes = float(np.sum(step_bytes))
    value = total_bytes / wall / 1e9
    # The roofline: bytes of the steps whose decode was timed over their mean time.
    achieved = float(np.mean([step_bytes[i] for i in timed])) / decode_avg_s / 1e9
    bytes_avg = float(np.mean(step_bytes))
    if unique_step_bytes:
        # Shared prompt blocks are read from HBM once; the roofline counts unique bytes.
        sc.extra["unique_kv_bytes_per_step"] = int(np.mean(unique_step_bytes))
        achieved = float(np.mean([unique_step_bytes[i] for i in timed])) / decode_avg_s / 1e9
    writes_copies = (write_copy_times(list(mark_ring.results().values()), sc, w)
                     if args.layout == "paged" else None)

    # The committed counter summaries describe the paged kernels at the workloads'
    # own block size (16) only.
    traffic = (counter_traffic(args.workload)
               if args.layout == "paged" and w.block_size == 16 else None)
    ceiling = None if args.no_read_probe else read_ceiling(dev)
    baseline = None
    if args.cpu_seconds > 0 and hasattr(w, "offsets") and args.layout == "paged":
        baseline = cpu_baseline(w, args.cpu_seconds)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} decode layer" + (f", block size {w.block_size}"
                                                    if w.block_size != 16 else ""),
            "arithmetic": "fp16 K/V (and q, except the tiny case) read, fp32 softmax and "
                          "accumulation",
            "timed_steps": [first_step, first_step + args.steps - 1],
            "num_seqs": sc.num_seqs, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": "f16",
            "q_dtype": np.dtype(w.q_dtype).name, "partition_size": plans[-1]["partition_size"],
            "prefix_groups": plans[-1].get("num_groups", 0),
            "group_pieces": plans[-1].get("num_group_items", 0),
            "kernel_policy": args.kernel_policy, "layout": args.layout,
            "schedule": "planner work list, largest piece first",
            "work_items": plans[-1]["num_items"], "waves_per_cu": plans[-1]["waves_per_cu"],
            "mean_context": round(float(np.mean(lengths)), 1),
            "kv_bytes_per_step": int(bytes_avg),
            **sc.extra,
        },
        "decode_us": round(decode_avg_s * 1e6, 2),
        "decode_timed_steps": len(timed),
        "decode_timing": f"kernel-level HIP events on every {every}th timed step",
        "decode_us_median": round(float(np.median(decode_ms)) * 1e3, 2),
        "decode_us_p10_p90": [round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                              round(float(np.percentile(decode_ms, 90)) * 1e3, 2)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "traffic_over_algorithmic": (round(traffic["traffic_bytes_per_launch"]
                                                       / traffic["algorithmic_bytes_per_launch"], 4)
                                                 if traffic else None),
                     "kernel": ("pa_decode_grouped (group pieces, remaining pieces, reduce)"
                                if plans[-1].get("num_groups", 0) else
                                "pa_decode (partition + reduce launches)"),
                     "measured_peak": ceiling,
                     "frac_of_measured": (round(achieved / ceiling["tile_gather"]["gbs"], 4)
                                          if ceiling else None)},
        "write_copy": writes_copies,
        "cpu_baseline": baseline,
        "gpu": GPU_INFO,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
