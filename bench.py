"""Benchmark of the batched verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replicas R] [--no-cpu-baseline]

Workload: the batch workload -- B=64 sequences, k=5 drafts, V=128256, bf16 target logits, fp32
draft probabilities, per-row temperature U[0.5, 1.2] (seeded synthetic inputs).  One step is
one specdec_verify call over that batch: row statistics of all 384 target rows, the accept
scan, and the residual / bonus draw.  Inputs are resident in HBM before timing starts; R
copies of them are rotated step by step so the 256 MB Infinity Cache cannot serve a step from
the previous one.

Timing: W untimed warmup steps, then REPEATS (5) timed repeats of exactly K steps each, every
repeat replayed from HIP graphs and bracketed by synchronisation and HIP events; the reported
step time is the median repeat's, and every repeat's figure and their spread are reported beside
it.  The other workloads are timed the same way (median of 5 repeats).

Prints ONE JSON line: verified draft positions per second (sum_b k_b per step / step time),
plus a roofline object for the streaming row-statistics kernel (algorithmic logit bytes per
launch / its HIP-event-timed duration, against the 8 TB/s HBM peak) and the fp64 CPU oracle's
rate on a bounded sample of the same workload.  ``dtype`` names the arithmetic the path computes
in (fp32 exponentials and sums; the accept tests and the draw's final scan in fp64); the target
logits it reads are bf16 (``config.logits_dtype``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec and HBM GB/s (% of peak), B=64 V=128256 k=5"
HBM_PEAK_GBS = 8000.0
REPEATS = 5
CPU_WORKER_CAP = 16   # the CPU share one GPU's host jobs may use, whatever the affinity mask shows
HOT_KERNEL = "stats_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stats_kernel_batch64_counters.txt")
# The streaming kernel's code: the kernel file and the device headers it is built from.
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_decoding_verification_specdec_amd", "csrc", f)
                  for f in ("kernels.hip", "kernels.h", "verify_dev.h", "wave_ops.h")]


def kernel_source_hash() -> str:
    """sha256[:16] of the streaming kernel's source code (its file and device headers, in that
    order): comments and blank lines stripped, so a comment edit does not invalidate a counter
    summary taken on the same code."""
    src = ""
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.strip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch of a kernel (``key``: the streaming kernel's line by default, or
    "accept_draw_kernel_hbm_bytes_per_launch") from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration it records), or None when
    the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    t = re.search(r"^" + re.escape(key) + r":\s*([0-9.eE+]+)", txt, flags=re.M)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


class HipEvents:
    """Raw hipEvent_t pairs from the HIP runtime (handed to the library, which records them on
    the kernel's own stream).  They are timing-only events created without the system-scope
    fence (hipEventDisableSystemFence): recording one then costs no L2 writeback / invalidate,
    which would otherwise be charged to the bracketed kernel.  Elapsed times are read only after
    a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = [(self._make(), self._make()) for _ in range(n)]

    def _make(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    def elapsed_ms(self, i: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), *self.pairs[i]) != 0:
            raise RuntimeError("hipEventElapsedTime failed (event not recorded?)")
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


_CPU_INP = None  # the batch the forked oracle workers read (inherited, not pickled)


def _cpu_shard(job):
    import oracle
    rows, reps = job
    for _ in range(reps):
        oracle.verify(_CPU_INP, rows=rows)
    return len(rows) * reps


def cpu_baseline(inp, budget_s: float = 6.0, parallel_s: float = 1.5):
    """The fp64 oracle (as it stands) on the same inputs, run before the GPU is touched so that
    worker processes can be forked: (i) one thread, whole batches repeated for about
    ``budget_s``; (ii) one forked worker per CPU of the affinity mask, at most CPU_WORKER_CAP,
    the batch's sequences split into one shard per worker, each worker repeating its shard for
    about ``parallel_s``.  ``cores`` is the number of workers used; ``affinity_cpus`` the size of
    the mask."""
    global _CPU_INP
    import multiprocessing

    import numpy as np

    import oracle
    positions = int(inp.draft_counts().sum())
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.verify(inp)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 200:
            break
    single = dict(value=positions * n / el, unit="positions/s", cores=1,
                  sample=f"{n} full oracle calls on the B=64 V=128256 k=5 batch ({el:.1f} s)")
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(CPU_WORKER_CAP, affinity))
    shards = [r for r in np.array_split(np.arange(inp.B), cores) if len(r)]
    reps = max(1, int(parallel_s / (el / n / len(shards))))
    _CPU_INP = inp
    with multiprocessing.get_context("fork").Pool(len(shards)) as pool:
        pool.map(_cpu_shard, [(r, 1) for r in shards])          # worker start-up, imports
        t0 = time.perf_counter()
        done = sum(pool.map(_cpu_shard, [(r, reps) for r in shards]))
        el_p = time.perf_counter() - t0
    _CPU_INP = None
    assert done == inp.B * reps
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=positions * reps / el_p, unit="positions/s", cores=len(shards),
                kind="oracle", cpu_model=model, affinity_cpus=affinity,
                worker_cap=CPU_WORKER_CAP,
                sample=f"{reps} passes over the B=64 V=128256 k=5 batch, its sequences split "
                       f"across {len(shards)} forked worker processes (one per host core, "
                       f"numpy fp64; {el_p:.1f} s)",
                single_core=single)


def algorithmic_bytes(inp, acc_np, all_rejected: bool = False):
    """Bytes the method must move per call: every used target row once, ids, q gathers,
    uniforms, temperatures, one draft row per rejected model-draft sampled sequence, outputs.
    ``all_rejected``: the upper bound, as if every sampled model-draft sequence were rejected."""
    import numpy as np
    kb = inp.draft_counts()
    sz = 2 if inp.logits_dtype == "bf16" else 4
    V = inp.V
    sampled = inp.temperature > 0
    onehot = np.zeros(inp.B, bool) if inp.draft_onehot is None else inp.draft_onehot.astype(bool)
    model = sampled & ~onehot
    rejected = np.ones(inp.B, bool) if all_rejected else (acc_np >= 0) & (acc_np < kb)
    logits = float(((kb + 1) * V * sz).sum())
    small = float((4 * kb + 4 * kb * model + 4 * (kb + 1) * sampled + 4 + 8 * (kb + 1) + 4).sum())
    draft_rows = float((rejected & model).sum() * 4 * V)
    return logits, logits + small + draft_rows


def _median_and_spread(us):
    """(median, {"repeats_us": each repeat's figure, "spread_pct": (max - min) / median})."""
    m = statistics.median(us)
    return m, {"repeats_us": [round(float(x), 4) for x in us],
               "spread_pct": (max(us) - min(us)) / m * 100.0}


def draft_row_bytes(inp, acc_np):
    """The draw kernel's algorithmic bytes: one fp32 draft row per rejected, sampled,
    model-draft sequence."""
    import numpy as np
    kb = inp.draft_counts()
    sampled = inp.temperature > 0
    onehot = np.zeros(inp.B, bool) if inp.draft_onehot is None else inp.draft_onehot.astype(bool)
    rejected = (acc_np >= 0) & (acc_np < kb)
    return float((rejected & sampled & ~onehot).sum() * 4 * inp.V)


def time_replayed(calls, steps, stream, repeats=REPEATS):
    """µs per call of ``calls`` (rotated) replayed from one HIP graph of ``steps`` calls: the
    median of ``repeats`` timed replays, each bracketed by synchronisation and events, after one
    untimed replay; returns (median, {"repeats_us", "spread_pct"})."""
    import torch
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            calls[i % len(calls)]()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    us = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / steps)
    return _median_and_spread(us)


def bench_ngram(dev, stream, steps=200, replicas=20, long=False):
    """The n-gram drafter on 512 histories of 4096-8192 tokens (V = 128256, n = 4..1, K = 8):
    history tokens scanned per second and the algorithmic bytes (4 per history token read,
    plus the proposals) against the HBM peak.  ``replicas`` copies (~340 MB) rotate so the
    Infinity Cache cannot hold them."""
    import numpy as np
    import torch
    from speculative_decoding_verification_specdec_amd import (specdec_ngram_propose,
                                                               specdec_ngram_workspace_size)
    from speculative_decoding_verification_specdec_amd.contexts import (ngram_long_workload,
                                                                        ngram_workload)
    h = ngram_long_workload() if long else ngram_workload()
    if long:
        replicas = 4        # 4 x 67 MB of histories
    K, n_min, n_max = 8, 1, 4
    ws = torch.empty(specdec_ngram_workspace_size(h.B, h.capacity), dtype=torch.uint8, device=dev)
    out = (torch.empty((h.B, K), dtype=torch.int32, device=dev),
           torch.empty(h.B, dtype=torch.int32, device=dev))
    calls = []
    for _ in range(replicas):
        t = torch.from_numpy(h.tokens).to(dev)
        ln = torch.from_numpy(h.lengths).to(dev)
        calls.append(lambda t=t, ln=ln: specdec_ngram_propose(t, ln, K, n_min=n_min, n_max=n_max,
                                                              out=out, workspace=ws))
    us, spread = time_replayed(calls, steps, stream)
    nd = out[1].cpu().numpy()
    toks = float(h.lengths.astype(np.int64).sum())
    nbytes = 4.0 * toks + 4.0 * h.B + 4.0 * h.B * (K + 1)
    return {
        "workload": (f"{h.B} token histories, length U{{{h.capacity // 2}..{h.capacity}}}, "
                     "V=128256, half the segments copied from earlier in the history; "
                     "n = 4..1, K = 8"),
        "us_per_call": us, "history_tokens_per_s": toks / (us * 1e-6),
        "algorithmic_GBps": nbytes / (us * 1e-6) / 1e9,
        "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "sequences_proposing": int((nd > 0).sum()), **spread,
    }


def bench_commit(dev, stream, steps=400):
    """The commit step on the ragged batch's shape: B = 512 sequences, K = 8, accept lengths
    U{0..8}, histories of capacity 8192 with lengths U{4096..8000}, both cache lengths rolled
    back, the packed stream and offsets written.  Latency-bound (a few KB move)."""
    import numpy as np
    import torch
    from speculative_decoding_verification_specdec_amd import specdec_commit
    B, K, cap = 512, 8, 8192
    rng = np.random.default_rng(21)
    acc = torch.from_numpy(rng.integers(0, K + 1, size=B).astype(np.int32)).to(dev)
    out = torch.from_numpy(rng.integers(0, 128256, size=(B, K + 1)).astype(np.int32)).to(dev)
    seq0 = rng.integers(4096, 8001, size=B).astype(np.int32)
    tokens = torch.zeros((B, cap), dtype=torch.int32, device=dev)
    seq = torch.from_numpy(seq0).to(dev)
    tkv = torch.from_numpy(seq0 + K).to(dev)
    dkv = torch.from_numpy(seq0 + K - 1).to(dev)
    packed = (torch.empty(B * (K + 1), dtype=torch.int32, device=dev),
              torch.empty(B + 1, dtype=torch.int32, device=dev))
    base = torch.from_numpy(seq0).to(dev)

    def call():
        # Lengths are reset by a device copy first so every call commits the same round.
        seq.copy_(base)
        specdec_commit(acc, out, seq, tokens=tokens, target_kv_len=tkv, draft_kv_len=dkv,
                       out=packed)
    us, spread = time_replayed([call], steps, stream)
    return {"workload": "B=512, K=8, accept lengths U{0..8}, history capacity 8192",
            "us_per_call_including_length_reset_copy": us,
            "sequences_per_s": B / (us * 1e-6), **spread}


def bench_workload(dev, stream, inp, description, steps=60, replicas=1):
    """Whole verify steps on another workload: verified positions/s and algorithmic GB/s.  One
    replica when a single step's logits already exceed twice the Infinity Cache, else
    ``replicas`` copies rotated step to step."""
    import torch
    from speculative_decoding_verification_specdec_amd import (inputs_to_device,
                                                               specdec_workspace_size)
    from speculative_decoding_verification_specdec_amd.binding import PreparedVerify
    B, K, V = inp.B, inp.K, inp.V
    ws = torch.zeros(specdec_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
    calls = []
    for _ in range(replicas):
        d = inputs_to_device(inp, dev)
        calls.append(PreparedVerify(d["logits"], d["draft_probs"], d["proposed"],
                                    d["temperature"], d["uniforms"],
                                    draft_onehot=d["draft_onehot"], num_draft=d["num_draft"],
                                    workspace=ws, out=calls[0].out if calls else None))
    us, spread = time_replayed(calls, steps, stream)
    acc = calls[0].out[0].cpu().numpy()
    _, nbytes = algorithmic_bytes(inp, acc)
    _, upper = algorithmic_bytes(inp, acc, all_rejected=True)
    positions = int(inp.draft_counts().sum())
    del d, calls, ws
    torch.cuda.empty_cache()
    return {"workload": description, "us_per_call": us,
            "verified_positions_per_s": positions / (us * 1e-6),
            "algorithmic_GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "upper_bound_bytes_frac_of_hbm_peak": upper / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mean_accept_len": float(acc[acc >= 0].mean()), "invalid_rows": int((acc < 0).sum()),
            "rejected_sequences": int(((acc >= 0) & (acc < inp.draft_counts())).sum()),
            **spread}


def bench_match(dev, stream, steps=300, replicas=6):
    """Sample-and-match verify on the same B=64, k=5, V=128256 bf16 batch: verified draft
    positions per second and the algorithmic bytes (every used logit row once, ids, uniforms,
    outputs; no draft row is read) against the HBM peak."""
    import torch
    from speculative_decoding_verification_specdec_amd import (inputs_to_device,
                                                               specdec_verify_match,
                                                               specdec_workspace_size)
    from speculative_decoding_verification_specdec_amd.inputs import batch64
    inp = batch64()
    B, K, V = inp.B, inp.K, inp.V
    ws = torch.zeros(specdec_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
    out = (torch.empty(B, dtype=torch.int32, device=dev),
           torch.empty((B, K + 1), dtype=torch.int32, device=dev),
           torch.empty((B, K + 1), dtype=torch.float32, device=dev))
    calls = []
    for _ in range(replicas):
        d = inputs_to_device(inp, dev)
        calls.append(lambda d=d: specdec_verify_match(d["logits"], d["proposed"], d["temperature"],
                                                      d["uniforms"], out=out, workspace=ws))
    us, spread = time_replayed(calls, steps, stream)
    acc = out[0].cpu().numpy()
    kb = inp.draft_counts()
    positions = int(kb.sum())
    nbytes = float(((kb + 1) * V * 2).sum() + (4 * kb + 4 * (kb + 1) + 4 + 8 * (kb + 1) + 4).sum())
    return {"workload": "batch64 (B=64, k=5, V=128256, bf16), sample-and-match verify",
            "us_per_call": us, "verified_positions_per_s": positions / (us * 1e-6),
            "algorithmic_GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mean_accept_len": float(acc.mean()), **spread}


def bench_greedy(dev, stream, steps=300, replicas=6):
    """Greedy verify (specdec_verify_greedy: every row at temperature 0, accept x_i iff it is
    the row's lowest argmax) on the same B=64, k=5, V=128256 bf16 batch: verified draft
    positions per second and the algorithmic bytes (every used logit row once, ids, outputs; no
    draft row, temperature or uniform is read) against the HBM peak."""
    import torch
    from speculative_decoding_verification_specdec_amd import (inputs_to_device,
                                                               specdec_verify_greedy,
                                                               specdec_workspace_size)
    from speculative_decoding_verification_specdec_amd.inputs import batch64
    inp = batch64()
    B, K, V = inp.B, inp.K, inp.V
    ws = torch.zeros(specdec_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
    out = (torch.empty(B, dtype=torch.int32, device=dev),
           torch.empty((B, K + 1), dtype=torch.int32, device=dev),
           torch.empty((B, K + 1), dtype=torch.float32, device=dev))
    calls = []
    for _ in range(replicas):
        d = inputs_to_device(inp, dev)
        calls.append(lambda d=d: specdec_verify_greedy(d["logits"], d["proposed"], out=out,
                                                       workspace=ws))
    us, spread = time_replayed(calls, steps, stream)
    acc = out[0].cpu().numpy()
    kb = inp.draft_counts()
    positions = int(kb.sum())
    nbytes = float(((kb + 1) * V * 2).sum() + (4 * kb + 8 * (kb + 1) + 4).sum())
    return {"workload": "batch64 (B=64, k=5, V=128256, bf16), greedy verify",
            "us_per_call": us, "verified_positions_per_s": positions / (us * 1e-6),
            "algorithmic_GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mean_accept_len": float(acc.mean()), **spread}


def bench_group_pipeline(dev, groups, steps=400, replicas=4):
    """The alternative of pipelining sequence groups across two streams, measured: the batch64
    batch split into ``groups`` groups of sequences, each its own specdec_verify call with its own
    workspace and output slices.  (a) the whole batch as one call; (b) the groups one after
    another on one stream; (c) the groups alternating between two streams, group g + 1 waiting
    (hipStreamWaitEvent) on an event recorded right after group g's streaming kernel, so that
    its streaming can overlap group g's draw; the first stream waits for the last group's.  All
    eager launches queued behind a spin kernel; µs per whole step; outputs compared bit for bit
    with (a)'s."""
    import ctypes

    import numpy as np
    import torch
    from speculative_decoding_verification_specdec_amd import (inputs_to_device,
                                                               specdec_workspace_size)
    from speculative_decoding_verification_specdec_amd.binding import PreparedVerify
    from speculative_decoding_verification_specdec_amd.inputs import batch64
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    inp = batch64()
    B, K, V = inp.B, inp.K, inp.V
    if B % groups:
        raise SystemExit(f"--group-pipeline: {groups} does not divide B = {B}")
    reps = [inputs_to_device(inp, dev) for _ in range(replicas)]
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()

    def outputs():
        return (torch.full((B,), -9, dtype=torch.int32, device=dev),
                torch.full((B, K + 1), -9, dtype=torch.int32, device=dev),
                torch.full((B, K + 1), -9.0, dtype=torch.float32, device=dev))

    def make(G, out):
        n = B // G
        wss = [torch.zeros(specdec_workspace_size(n, K, V), dtype=torch.uint8, device=dev)
               for _ in range(G)]
        calls = []
        for d in reps:
            cs = []
            for g in range(G):
                sl = slice(g * n, (g + 1) * n)
                cs.append(PreparedVerify(d["logits"][sl], d["draft_probs"][sl], d["proposed"][sl],
                                         d["temperature"][sl], d["uniforms"][sl],
                                         out=tuple(t[sl] for t in out), workspace=wss[g]))
            calls.append(cs)
        return calls

    def run(G, pipelined):
        out = outputs()
        calls = make(G, out)
        ev = HipEvents(steps * G)
        join = HipEvents(steps)
        for i in range(10):
            for c in calls[i % replicas]:
                c(stream=sA)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(sA):
            torch.cuda._sleep(int(3e8))
            e0.record(sA)
        for i in range(steps):
            cs = calls[i % replicas]
            if not pipelined:
                for c in cs:
                    c(stream=sA)
                continue
            streams = [sA, sB]
            for g, c in enumerate(cs):
                s = streams[g % 2]
                if g > 0:
                    hip.hipStreamWaitEvent(s.cuda_stream, ev.pairs[i * G + g - 1][1], 0)
                c(stream=s, hot_events=ev.pairs[i * G + g])
            if (G - 1) % 2:
                hip.hipEventRecord(join.pairs[i][0], sB.cuda_stream)
                hip.hipStreamWaitEvent(sA.cuda_stream, join.pairs[i][0], 0)
        e1.record(sA)
        torch.cuda.synchronize()
        ev.close()
        join.close()
        return e0.elapsed_time(e1) * 1e3 / steps, [t.cpu().numpy() for t in out]

    whole_us, ref = run(1, False)
    serial_us, o1 = run(groups, False)
    piped_us, o2 = run(groups, True)
    same = all(np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
               for o in (o1, o2) for a, b in zip(o, ref))
    return {"workload": f"batch64 (B=64, k=5, V=128256, bf16) in {groups} groups of "
                        f"{B // groups} sequences", "steps": steps,
            "whole_batch_one_call_us": whole_us, "groups_one_stream_us": serial_us,
            "groups_pipelined_two_streams_us": piped_us, "outputs_identical": bool(same)}


def bench_telemetry(dev, stream, steps=400):
    """Telemetry update of a B=512, K=8 batch into 4 routes, and applying a 4-route plan."""
    import numpy as np
    import torch
    from speculative_decoding_verification_specdec_amd import (specdec_apply_k,
                                                               specdec_telemetry_update,
                                                               telemetry_counters)
    B, K = 512, 8
    rng = np.random.default_rng(22)
    nd = torch.from_numpy(rng.integers(1, K + 1, size=B).astype(np.int32)).to(dev)
    acc = torch.from_numpy((rng.random(B) * (nd.cpu().numpy() + 1)).astype(np.int32)).to(dev)
    route = torch.from_numpy(rng.integers(0, 4, size=B).astype(np.int32)).to(dev)
    cnt = telemetry_counters(4, dev)
    table = torch.tensor([3, 5, 8, 2], dtype=torch.int32, device=dev)
    nd2 = nd.clone()
    us_t, spread_t = time_replayed([lambda: specdec_telemetry_update(cnt, acc, num_draft=nd,
                                                                     route=route, K=K)],
                                   steps, stream)
    us_a, spread_a = time_replayed([lambda: specdec_apply_k(nd2, table, route=route)], steps,
                                   stream)
    return {"workload": "B=512, K=8, 4 routes", "update_us": us_t, "apply_k_us": us_a,
            "update_spread_pct": spread_t["spread_pct"],
            "apply_k_spread_pct": spread_a["spread_pct"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["auto", "one_launch", "quad"], default="auto",
                    help="streaming path of the headline call: the default three launches, or one of "
                         "the one-launch alternatives kept for comparison (workgroups per 8192-token "
                         "tile, or four workgroups per sequence)")
    ap.add_argument("--cpu-budget", type=float, default=6.0,
                    help="seconds of the single-thread oracle leg")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the drafter / commit / match-mode / telemetry measurements")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the large-batch and ragged workloads")
    ap.add_argument("--small-vocab-only", action="store_true",
                    help="only the small-vocabulary-path workloads (tiny vocabulary call, one-round "
                         "latency): for profiling that kernel")
    ap.add_argument("--group-pipeline", type=int, default=0, metavar="G",
                    help="only measure the two-stream sequence-group pipelining alternative "
                         "(batch64 in G groups) against the whole-batch call")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 20 device-to-device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verify step shards by sequence with no "
              "communication, so only --gpus 1 is supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from speculative_decoding_verification_specdec_amd import (inputs_to_device, specdec_verify,
                                                               specdec_workspace_size)
    from speculative_decoding_verification_specdec_amd.inputs import batch64

    cpu = None
    if not (args.no_cpu_baseline or args.copy_calibration or args.small_vocab_only
            or args.group_pipeline):
        # Before any GPU call: the all-core leg forks worker processes.
        print("[bench] timing the CPU oracle on the batch", file=sys.stderr, flush=True)
        cpu = cpu_baseline(batch64(), args.cpu_budget)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters calibrate the
        # hot kernel's (bytes read = bytes written = MIB MiB per copy).
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 20}))
        return
    from speculative_decoding_verification_specdec_amd.binding import (SPECDEC_PATH_AUTO,
                                                                       SPECDEC_PATH_ONE_LAUNCH,
                                                                       SPECDEC_PATH_QUAD,
                                                                       PreparedVerify)
    path = {"one_launch": SPECDEC_PATH_ONE_LAUNCH, "quad": SPECDEC_PATH_QUAD}.get(args.path,
                                                                               SPECDEC_PATH_AUTO)
    if args.group_pipeline:
        print(json.dumps({"group_pipeline": bench_group_pipeline(dev, args.group_pipeline)}))
        return
    if args.small_vocab_only:
        from speculative_decoding_verification_specdec_amd.inputs import tiny_vocab
        stream = torch.cuda.Stream()
        print(json.dumps({
            "tiny_vocab": bench_workload(dev, stream, tiny_vocab(),
                                         "B=100000, k=4, V=32, fp32; 4 replicas rotated",
                                         steps=100, replicas=4),
            "tiny_vocab_one_round": bench_workload(dev, stream, tiny_vocab(rounds=1),
                                                   "B=1, k=4, V=32, fp32", steps=400)}))
        return

    print("[bench] generating the B=64 V=128256 k=5 batch", file=sys.stderr, flush=True)
    inp = batch64()
    B, K, V = inp.B, inp.K, inp.V
    ws = torch.zeros(specdec_workspace_size(B, K, V), dtype=torch.uint8, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    prb = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
    calls = []
    for _ in range(args.replicas):
        d = inputs_to_device(inp, dev)
        calls.append(PreparedVerify(d["logits"], d["draft_probs"], d["proposed"],
                                    d["temperature"], d["uniforms"],
                                    draft_onehot=d["draft_onehot"], num_draft=d["num_draft"],
                                    out=(acc, tok, prb), workspace=ws, path=path))
    R = len(calls)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    print(f"[bench] warmup {args.warmup}, timed {args.steps}", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            calls[i % R]()
    torch.cuda.synchronize()

    # One HIP graph holds R consecutive steps (one per input replica); a second holds the
    # remainder, so the timed region replays exactly `steps` steps with no host launch gaps.
    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                calls[i % R]()
        return g
    full, rem = divmod(args.steps, R)
    g_full = capture(R) if full else None
    g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()
    if g_full is not None:
        g_full.replay()                      # one untimed replay of each graph
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()

    # Timed regions: REPEATS repeats of exactly `steps` whole steps, each bracketed by
    # synchronisation and HIP events; the median repeat is the reported step time.
    rep_ms, rep_wall = [], []
    for _ in range(REPEATS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(full):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        rep_wall.append(time.perf_counter() - w0)
        rep_ms.append(e0.elapsed_time(e1) / args.steps)
    ms_per_step, spread = _median_and_spread(rep_ms)
    spread["repeats_us"] = [round(x * 1e3, 4) for x in rep_ms]
    wall = statistics.median(rep_wall)

    # The same steps launched eagerly, with HIP events recorded by the library around the
    # streaming row-statistics kernel of each step.  A spin kernel in front lets the host
    # queue every launch before the GPU reaches them, so the events bracket kernel time only.
    # The kernels after it (accept scan, draw sums, pick) are bracketed by a second pair.
    hot, drw = HipEvents(args.steps), HipEvents(args.steps)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(2e8))
        for i in range(args.steps):
            calls[i % R](hot_events=hot.pairs[i], draw_events=drw.pairs[i])
    torch.cuda.synchronize()
    hot_ms = sum(hot.elapsed_ms(i) for i in range(args.steps)) / args.steps
    draw_ms = (sum(drw.elapsed_ms(i) for i in range(args.steps)) / args.steps
               if args.path == "auto" else None)
    hot.close()
    drw.close()

    acc_np = acc.cpu().numpy()
    assert (acc_np >= 0).all(), "invalid rows in the benchmark batch"
    logit_bytes, call_bytes = algorithmic_bytes(inp, acc_np)
    _, upper_bytes = algorithmic_bytes(inp, acc_np, all_rejected=True)
    positions = int(inp.draft_counts().sum())
    value = positions / (ms_per_step * 1e-3)
    achieved = logit_bytes / (hot_ms * 1e-3) / 1e9
    # The counters summarised under profiles/ are the default path's streaming kernel's.
    traffic = measured_traffic() if args.path == "auto" else None
    draft_bytes = draft_row_bytes(inp, acc_np)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "batch64: B=64 sequences, k=5 drafts, V=128256, bf16 target logits "
                        "~N(0,3^2), fp32 draft probs from 0.8z+N(0,1.5^2), T~U[0.5,1.2]",
            "global_batch": B, "k": K, "vocab": V, "logits_dtype": "bf16",
            "replicas_rotated": args.replicas,
        },
        "roofline": {
            # On the one-launch alternatives the timed kernel does the whole call.
            "kernel": {"auto": HOT_KERNEL, "one_launch": "verify_kernel",
                       "quad": "quad_verify_kernel"}[args.path],
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel_us": hot_ms * 1e3,
            "bytes_per_launch": logit_bytes,
        },
        # The draw kernel (accept scan, draw sums and the pick, one launch here): its
        # algorithmic bytes are the rejected rows' draft probabilities (the target rows it
        # re-reads to form p - q are not counted).
        "roofline_draw": None if draw_ms is None else {
            "kernel": "accept_draw_kernel",
            "bound": "hbm",
            "achieved": draft_bytes / (draw_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": draft_bytes / (draw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic("accept_draw_kernel_hbm_bytes_per_launch"),
            "kernel_us": draw_ms * 1e3,
            "bytes_per_launch": draft_bytes,
        },
        "whole_step": {
            "us": ms_per_step * 1e3,
            "wall_us": wall / args.steps * 1e6,
            "algorithmic_bytes": call_bytes,
            "algorithmic_GBps": call_bytes / (ms_per_step * 1e-3) / 1e9,
            "frac_of_hbm_peak": call_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "upper_bound_bytes": upper_bytes,
            "upper_bound_frac_of_hbm_peak":
                upper_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "rejected_sequences": int((acc_np < K).sum()),
            "repeats": REPEATS, **spread,
        },
    }
    if not args.no_next_rows:
        print("[bench] n-gram drafter", file=sys.stderr, flush=True)
        res["next_rows"] = {"ngram_propose": bench_ngram(dev, stream),
                            "ngram_propose_long": bench_ngram(dev, stream, long=True)}
        print("[bench] commit", file=sys.stderr, flush=True)
        res["next_rows"]["commit"] = bench_commit(dev, stream)
        print("[bench] sample-and-match verify", file=sys.stderr, flush=True)
        res["next_rows"]["verify_match"] = bench_match(dev, stream)
        print("[bench] greedy verify", file=sys.stderr, flush=True)
        res["next_rows"]["verify_greedy"] = bench_greedy(dev, stream)
        print("[bench] telemetry", file=sys.stderr, flush=True)
        res["next_rows"]["telemetry"] = bench_telemetry(dev, stream)
    if not args.no_other_workloads:
        from speculative_decoding_verification_specdec_amd.inputs import (large_batch_deep,
                                                                           ragged_mixed,
                                                                           single_sequence,
                                                                           tiny_vocab)
        print("[bench] large batch, deep draft", file=sys.stderr, flush=True)
        res["other_workloads"] = {"large_batch_deep": bench_workload(
            dev, stream, large_batch_deep(),
            "B=256, k=8, V=152064, bf16 logits ~N(0,4^2) + 8 on 1% of entries, 25% greedy rows")}
        print("[bench] large batch, deep calibrated draft", file=sys.stderr, flush=True)
        res["other_workloads"]["large_batch_deep_calibrated"] = bench_workload(
            dev, stream, large_batch_deep(calibrated=True),
            "large_batch_deep with draft noise 0.3 (acceptance ~0.7): the k=8 bonus path")
        print("[bench] ragged mixed drafters", file=sys.stderr, flush=True)
        res["other_workloads"]["ragged_mixed"] = bench_workload(
            dev, stream, ragged_mixed(),
            "B=512, k_b ~ U{1..8} padded to 8, V=128256, bf16; half n-gram (one-hot) rows")
        print("[bench] single-sequence latency", file=sys.stderr, flush=True)
        res["latency"] = {
            "single_sequence": bench_workload(
                dev, stream, single_sequence(),
                "B=1, k=4, V=32000, fp32 logits ~N(0,3^2), T=0.7: one call's latency", steps=400),
            "tiny_vocab_one_round": bench_workload(
                dev, stream, tiny_vocab(rounds=1),
                "B=1, k=4, V=32, fp32: one round's latency", steps=400)}
        print("[bench] tiny vocabulary, 1e5 rounds in one call", file=sys.stderr, flush=True)
        res["other_workloads"]["tiny_vocab"] = bench_workload(
            dev, stream, tiny_vocab(),
            "B=100000 rounds of one sequence, k=4, V=32, fp32 logits ~N(0,2^2), q = softmax of "
            "logits + N(0,1), T=1: one call (eight sequences per wave); 4 replicas rotated",
            steps=100, replicas=4)
        print("[bench] batch, calibrated drafter", file=sys.stderr, flush=True)
        res["other_workloads"]["batch64_calibrated"] = bench_workload(
            dev, stream, batch64(calibrated=True),
            "batch64 with draft noise 0.5 and q softmaxed at the row's temperature (acceptance "
            "0.6-0.8); 6 replicas rotated", steps=300, replicas=6)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
