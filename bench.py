"""Benchmark of the sparse MLA hot path on one MI355X.

A step is one pass of the whole path over one batch: sa_layer_stack over the
decode workload of 16 sequences with 65,536..131,072 cached tokens each (seeded
ragged lengths) and a 4-layer IndexShare group [full, shared, shared, shared]:
indexer score -> exact top-2048 -> sparse MLA + W_UV on the full layer, sparse
MLA + W_UV with the reused selection on the three shared layers.

Output: one JSON line.  `value` is decode queries/s of back-to-back HIP-graph
replays of the step with inputs resident in HBM; the steps rotate through two
independent input sets, so no step finds the previous step's data in the 256 MB
last-level cache.  `roofline` describes the dominant kernel (the decode
indexer, ~2/3 of the step's bytes), timed with HIP events recorded on the
library's stream around that kernel in eager steps over the same input sets.  `prefill_indexer` is the chunked-prefill indexer
(4096 queries over 131,072 keys) in TFLOP/s.  `cache_write` is the cache-write step
(`sa_cache_write`) for one 4096-token prefill chunk of one layer, in GB/s of
algorithmic bytes against the HBM peak.  `cpu_baseline` is the CPU oracle
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c2", choices=["c0", "c1", "c2", "c3", "c4"],
                    help="c3 times the whole chunked-prefill stack; its dominant kernel is the MFMA-bound indexer")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill indexer and cache-write measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-query", action="store_true", help="skip the query-side (projection and absorption) legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache leg of the decode step")
    ap.add_argument("--cpu-sample", type=int, default=16, help="queries in the CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="repeat the CPU sample for at least this long")
    ap.add_argument("--copies", type=int, default=2,
                    help="independent input sets the timed steps rotate through, so one step's data is not "
                         "still in the 256 MB last-level cache when the next step reads it")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (reads and writes that many bytes): the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_decode_c2_traffic.md")
INDEXER_SOURCES = [os.path.join(ROOT, "sparse_attention_relu_amd", "csrc", f)
                   for f in ("indexer.hip", "sa_common.h")]


def indexer_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in INDEXER_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the decode indexer from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, scaled by a plain copy of known size; None
    when the summary is missing, is for another workload, or was taken on
    different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            fields = dict(line.split(":", 1) for line in fh.read().splitlines() if line.startswith("- ") and ":" in line)
    except OSError:
        return None
    fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("workload") != workload or fields.get("source_sha256") != indexer_source_hash():
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_bytes(wl, k=2048):
    """Algorithmic HBM bytes of one step: every input read once, every output
    written once (intermediate scores and partial results excluded)."""
    n_q = wl.n_q
    keys = sum(p + 1 for p in wl.q_pos)
    idx_bytes = keys * 256 + n_q * (32 * 128 * 2 + 32 * 4)
    k_eff = sum(min(k, p + 1) for p in wl.q_pos)
    per_layer = k_eff * 576 * 2 + n_q * 64 * 576 * 2 + 64 * 256 * 512 * 2 + n_q * 64 * 256 * 2
    n_full = sum(wl.full)
    return idx_bytes * n_full + per_layer * wl.n_layers + n_full * n_q * k * 4, idx_bytes


def layer_attn_bytes(wl, k=2048):
    """Algorithmic bytes of one layer's sparse attention + W_UV: the selected
    rows, the absorbed queries, W_UV and the output (indices excluded)."""
    k_eff = sum(min(k, p + 1) for p in wl.q_pos)
    return k_eff * 576 * 2 + wl.n_q * 64 * 576 * 2 + 64 * 256 * 512 * 2 + wl.n_q * 64 * 256 * 2


def cpu_baseline(b, wl, n_sample, min_seconds):
    """The CPU oracle (NumPy, float64) on the first n_sample queries: indexer
    scores and top-k for the full layer, sparse MLA + W_UV for all layers.
    Gathering the selected rows from device memory is done outside the timer."""
    import numpy as np
    import torch
    from oracle import ref
    from sparse_attention_relu_amd.synth import to_numpy

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    S = list(range(min(n_sample, wl.n_q)))
    seq = [wl.q_seq[t] for t in S]
    pos = [wl.q_pos[t] for t in S]
    starts = wl.seq_start
    L0 = b.layers[0]
    kparts = [to_numpy(L0.k_idx[starts[s]:starts[s] + p + 1]) for s, p in zip(seq, pos)]
    loc_start = np.concatenate([[0], np.cumsum([len(x) for x in kparts])[:-1]]).astype(np.int64)
    k_cpu = np.concatenate(kparts)
    q_cpu, w_cpu = to_numpy(L0.q_idx[S]), to_numpy(L0.w[S])
    t0 = time.perf_counter()
    sc = ref.indexer_scores(q_cpu, w_cpu, k_cpu, loc_start, np.arange(len(S)), np.array(pos))
    idx = ref.topk_select_rows(sc, np.array(pos), 2048)
    t_idx = time.perf_counter() - t0
    t_mla = 0.0
    mla_inputs = []
    for L in b.layers:
        rows, qa = [], to_numpy(L.q_abs[S])
        for j, t in enumerate(S):
            sel = torch.as_tensor(idx[j][idx[j] >= 0], device=L.kv.device) + starts[seq[j]]
            rows.append(to_numpy(L.kv[sel]))
        k_loc = np.concatenate(rows)
        st = np.concatenate([[0], np.cumsum([len(r) for r in rows])[:-1]]).astype(np.int64)
        loc_idx = np.full(idx.shape, -1)
        for j in range(len(S)):
            n = len(rows[j])
            loc_idx[j, :n] = np.arange(n)
        mla_inputs.append((qa, k_loc, st, loc_idx, to_numpy(L.w_uv)))
    reps = 0
    while True:
        reps += 1
        if reps > 1:
            t0 = time.perf_counter()
            sc = ref.indexer_scores(q_cpu, w_cpu, k_cpu, loc_start, np.arange(len(S)), np.array(pos))
            ref.topk_select_rows(sc, np.array(pos), 2048)
            t_idx += time.perf_counter() - t0
        for qa, k_loc, st, loc_idx, wuv in mla_inputs:
            t0 = time.perf_counter()
            ref.sparse_mla(qa, k_loc, st, np.arange(len(S)), loc_idx, wuv, wl.scale)
            t_mla += time.perf_counter() - t0
        if t_idx + t_mla >= min_seconds or reps >= 100:
            break
    total = t_idx + t_mla
    return {"value": reps * len(S) / total, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(S)} of {wl.n_q} queries of the same workload through all {wl.n_layers} layers, "
                      f"repeated {reps}x (indexer + top-k {t_idx:.2f} s, attention {t_mla:.2f} s); "
                      f"gathering rows from device memory untimed",
            "seconds": round(total, 3)}


def cache_write_leg(seed, reps=15, warmup=5, n=4096, rows=131072):
    """sa_cache_write on one 4096-token prefill chunk (positions 126,976..
    131,071 of a 131,072-row cache, with indexer keys), HIP-event median."""
    import torch
    from sparse_attention_relu_amd import api, synth
    dev = torch.device("cuda:0")
    g = synth._gen(dev, seed, 0, 7)
    kv_a = synth._randn((n, 576), g, dev, std=1.0, dtype=torch.bfloat16)
    k_raw = synth._randn((n, 128), g, dev, std=1.0, dtype=torch.bfloat16)
    gamma = torch.ones(512, dtype=torch.bfloat16, device=dev)
    ln_w = torch.ones(128, dtype=torch.bfloat16, device=dev)
    ln_b = torch.zeros(128, dtype=torch.bfloat16, device=dev)
    pos = torch.arange(rows - n, rows, dtype=torch.int32, device=dev)
    dst = pos.to(torch.int64)
    kv_cache = torch.empty((rows, 576), dtype=torch.bfloat16, device=dev)
    k_cache = torch.empty((rows, 128), dtype=torch.bfloat16, device=dev)
    call = lambda st=None: api.cache_write(kv_a, gamma, pos, dst, kv_cache, k_raw, ln_w, ln_b, k_cache, stream=st)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, c in ev:
        a.record(s)
        call(s)
        c.record(s)
    torch.cuda.synchronize()
    spread = sorted(a.elapsed_time(c) for a, c in ev)
    ms = spread[len(ev) // 2]
    # inputs read and rows written (bf16), positions and row indices, weights
    nbytes = n * (576 + 128) * 2 * 2 + n * (4 + 8) + (512 + 2 * 128) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "cache_write_4096_tokens_at_126976", "ms": round(ms, 5), "bytes": nbytes,
            "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
            "ms_min": round(spread[0], 5), "ms_max": round(spread[-1], 5),
            "timing": "median of %d HIP-event-timed launches" % reps}


def prefill_indexer(seed, reps=9, warmup=20):
    import torch
    from sparse_attention_relu_amd import api, synth
    wl = synth.workload("c3")
    dev = torch.device("cuda:0")
    g = synth._gen(dev, seed, 0, 4)
    q = synth._randn((wl.n_q, 32, 128), g, dev, std=1 / 128 ** 0.5, dtype=torch.bfloat16)
    w = synth._randn((wl.n_q, 32), synth._gen(dev, seed, 0, 5), dev, std=1 / 32 ** 0.5)
    _, kI = synth.law_rows(wl.seq_lens, synth._gen(dev, seed, 0, 2), synth._gen(dev, seed, 0, 6), dev)
    seq_start = torch.zeros(1, dtype=torch.int64, device=dev)
    seq_len = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    q_seq = torch.zeros(wl.n_q, dtype=torch.int32, device=dev)
    q_pos = torch.tensor(wl.q_pos, dtype=torch.int32, device=dev)
    scores = torch.empty((wl.n_q, wl.ld), dtype=torch.float32, device=dev)
    # the clocks settle over the first 10-15 launches of this 4 ms kernel
    for _ in range(warmup):
        api.indexer_score(q, w, kI, seq_start, seq_len, q_seq, q_pos, wl.ld, scores=scores)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, c in ev:
        a.record(s)
        api.indexer_score(q, w, kI, seq_start, seq_len, q_seq, q_pos, wl.ld, scores=scores, stream=s)
        c.record(s)
    # the shader clock level while the launches run (they are queued; the
    # host samples the driver's table during their ~30 ms)
    sclk = []
    for _ in range(6):
        time.sleep(0.004)
        cur, _top = gpu_sclk_mhz()
        if cur is not None:
            sclk.append(cur)
    torch.cuda.synchronize()
    spread = sorted(a.elapsed_time(c) for a, c in ev)
    ms = spread[len(ev) // 2]
    causal_flops = sum(2.0 * 32 * 128 * (p + 1) for p in wl.q_pos)
    tflops = causal_flops / (ms * 1e-3) / 1e12
    return {"workload": wl.name, "tflops": round(tflops, 1), "ms": round(ms, 4), "unit": "TFLOP/s",
            "flops": causal_flops, "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "peak": BF16_PEAK_TFLOPS, "ms_min": round(spread[0], 5), "ms_max": round(spread[-1], 5),
            "sclk_mhz_during": sorted(sclk)[len(sclk) // 2] if sclk else None,
            "timing": "median of %d HIP-event-timed launches" % reps}


def query_side_leg(seed, n, reps=15, warmup=10):
    """sa_q_project + sa_q_absorb for n tokens (random-init weights of the
    model's shapes), HIP-event medians per call.  Algorithmic bytes: every
    weight and activation read once, every output written once; FLOPs: the
    two contractions."""
    import math
    import torch
    from sparse_attention_relu_amd import api
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed + 17)
    bf = lambda x: x.to(torch.bfloat16).contiguous()
    w_qb = bf(torch.randn((64 * 256, 2048), generator=g, device=dev) / math.sqrt(2048))
    w_uk_t = bf(torch.randn((64, 512, 192), generator=g, device=dev) / math.sqrt(192 * 576))
    w_iq = bf(torch.randn((32 * 128, 2048), generator=g, device=dev) / math.sqrt(2048 * 128))
    w_iw = bf(torch.randn((32, 2048), generator=g, device=dev) / math.sqrt(2048 * 32))
    c = bf(torch.randn((n, 2048), generator=g, device=dev))
    pos = torch.arange(131072 - n, 131072, dtype=torch.int32, device=dev)
    q = torch.empty((n, 64, 256), dtype=torch.bfloat16, device=dev)
    qi = torch.empty((n, 32, 128), dtype=torch.bfloat16, device=dev)
    w = torch.empty((n, 32), dtype=torch.float32, device=dev)
    qa = torch.empty((n, 64, 576), dtype=torch.bfloat16, device=dev)
    proj = lambda st=None: api.q_project(c, w_qb, pos, w_iq=w_iq, w_iw=w_iw, q=q, q_idx=qi, w=w, stream=st)
    absorb = lambda st=None: api.q_absorb(q, w_uk_t, q_abs=qa, stream=st)
    for _ in range(warmup):
        proj()
        absorb()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    times = {}
    for name, fn in (("q_project", proj), ("q_absorb", absorb)):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, e in ev:
            a.record(s)
            fn(s)
            e.record(s)
        torch.cuda.synchronize()
        times[name] = sorted(a.elapsed_time(e) for a, e in ev)[reps // 2]
    rows = 64 * 256 + 32 * 128 + 32
    b_proj = rows * 2048 * 2 + n * 2048 * 2 + n * (64 * 256 * 2 + 32 * 128 * 2 + 32 * 4) + n * 4
    b_abs = 64 * 512 * 192 * 2 + n * 64 * 256 * 2 + n * 64 * 576 * 2
    f_proj = 2.0 * n * rows * 2048
    f_abs = 2.0 * n * 64 * 192 * 512
    out = {"tokens": n, "unit_time": "ms", "timing": "median of %d HIP-event-timed calls" % reps}
    for name, ms, nb, fl in (("q_project", times["q_project"], b_proj, f_proj),
                             ("q_absorb", times["q_absorb"], b_abs, f_abs)):
        gbs = nb / (ms * 1e-3) / 1e9
        tfl = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 5), "bytes": nb, "flops": fl, "gbs": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "tflops": round(tfl, 1),
                     "frac_of_bf16_peak": round(tfl / BF16_PEAK_TFLOPS, 4)}
    return out


def step_bytes_fp8(wl, k=2048):
    """step_bytes for FP8 caches: 128 code bytes + a 4-byte scale per indexer
    key, 576 + 4 per gathered row; queries, W_UV and outputs unchanged."""
    n_q = wl.n_q
    keys = sum(p + 1 for p in wl.q_pos)
    idx_bytes = keys * 132 + n_q * (32 * 128 * 2 + 32 * 4)
    k_eff = sum(min(k, p + 1) for p in wl.q_pos)
    per_layer = k_eff * 580 + n_q * 64 * 576 * 2 + 64 * 256 * 512 * 2 + n_q * 64 * 256 * 2
    n_full = sum(wl.full)
    return idx_bytes * n_full + per_layer * wl.n_layers + n_full * n_q * k * 4


def fp8_leg(batches, wl, steps, warmup):
    """The same step with both caches stored as FP8 (quantized on the GPU from
    the bf16 inputs), HIP-graph replays rotating through the input sets."""
    import torch
    from sparse_attention_relu_amd import api, synth
    stacks = []
    for b in batches:
        layers = []
        for L in b.layers:
            kv8, kvs = api.quantize_rows_fp8(L.kv)
            L8 = synth.LayerInputs(q_abs=L.q_abs, kv=kv8, w_uv=L.w_uv, q_idx=L.q_idx, w=L.w, kv_scale=kvs)
            if L.k_idx is not None:
                L8.k_idx, L8.k_scale = api.quantize_rows_fp8(L.k_idx)
            layers.append(L8)
        stacks.append(api.LayerStack(layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full))
        stacks[-1]()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for st_ in stacks:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                st_()
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    spread = replay_spread(graphs, steps)
    nb = step_bytes_fp8(wl)
    gbs = nb / (ms * 1e-3) / 1e9
    return {"workload": wl.name + "_fp8_caches", "ms_per_step": round(ms, 5),
            "value": round(wl.n_q / (ms * 1e-3), 1), "unit": "queries/s", "step_bytes": nb,
            "hbm_gbs_step": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "replay_ms": spread, "timing": "%d graph replays after %d warm-up" % (steps, warmup)}


def replay_spread(graphs, n):
    """Median, min and max of n graph replays, each between its own pair of
    HIP events (a second pass after the timed region; the headline figure is
    the wall-clock mean of the timed region)."""
    import torch
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, c) in enumerate(ev):
        a.record(s)
        graphs[i % len(graphs)].replay()
        c.record(s)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(c) for a, c in ev)
    return {"median": round(ms[len(ms) // 2], 5), "min": round(ms[0], 5), "max": round(ms[-1], 5), "n": n,
            "timing": "HIP events around each replay"}


def stage_fractions(kern_ms, eager_ms):
    rest = max(eager_ms - kern_ms["indexer"] - kern_ms["topk"], 0.0)
    return {"indexer": round(kern_ms["indexer"] / eager_ms, 4), "topk": round(kern_ms["topk"] / eager_ms, 4),
            "attention_all_layers": round(rest / eager_ms, 4), "attention_all_layers_ms": round(rest, 5)}


def gpu_sclk_mhz():
    """(current, highest) shader clock levels in MHz from the driver's sysfs
    table (the current level is marked '*'), or (None, None) where it cannot
    be read."""
    import glob
    import re
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                lines = fh.read().splitlines()
        except OSError:
            continue
        cur, levels = None, []
        for line in lines:
            m = re.search(r"(\d+)\s*mhz", line.lower())
            if not m:
                continue
            levels.append(int(m.group(1)))
            if line.rstrip().endswith("*"):
                cur = int(m.group(1))
        if levels:
            return cur, max(levels)
    return None, None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def environment(torch, sclk_after):
    p = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "sclk_mhz_after_timed_region": sclk_after[0], "sclk_mhz_top_level": sclk_after[1],
            "rocm": rocm, "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu_model()}


class HipEvents:
    """Raw hipEvents (the library records them on its stream)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the sharding plan is in DESIGN.md); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_attention_relu_amd import api, synth

    dev = torch.device("cuda:0")
    wl = synth.workload(args.workload, seed=args.seed)
    print(f"[bench] generating {wl.name}: {wl.n_q} queries, {wl.total_tokens} cached tokens, {wl.n_layers} layers",
          file=sys.stderr, flush=True)
    batches, stacks = [], []
    for c in range(max(1, args.copies)):
        b = synth.make_batch(wl, dev, seed=args.seed + c)
        batches.append(b)
        stacks.append(api.LayerStack(b.layers, b.seq_start, b.seq_len, b.q_seq, b.q_pos, wl.ld, full=wl.full))
        stacks[-1]()
    b = batches[0]
    torch.cuda.synchronize()

    # one HIP graph per input set, captured on a side stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for st_ in stacks:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                st_()
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)        # elementwise: reads and writes calib_copy_mib MiB
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    sclk_after = gpu_sclk_mhz()
    print(f"[bench] timed {args.steps} graph replays: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    replay_ms = replay_spread(graphs, args.steps)

    # Per-kernel HIP-event timing: eager steps rotating through the same input
    # sets, issued back to back (each step has its own events) and read after
    # one synchronisation, so the GPU runs them as it runs the graph replays.
    s = torch.cuda.current_stream()
    names = ["indexer", "topk", "attn"]
    acc = {n: [] for n in names}
    steps_ms = []
    n_ev = max(6, min(args.steps, 20))
    hev = HipEvents(6 * n_ev)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    for i in range(n_ev):
        step_ev[i][0].record(s)
        stacks[i % len(stacks)](events=hev.ev[6 * i:6 * i + 6], stream=s)
        step_ev[i][1].record(s)
    torch.cuda.synchronize()
    for i in range(n_ev):
        for j, n in enumerate(names):
            acc[n].append(hev.ms(6 * i + 2 * j, 6 * i + 2 * j + 1))
        steps_ms.append(step_ev[i][0].elapsed_time(step_ev[i][1]))
    hev.close()
    kern_ms = {n: sum(v) / len(v) for n, v in acc.items()}
    eager_ms = sum(steps_ms) / len(steps_ms)
    total_bytes, idx_bytes = step_bytes(wl)
    attn_bytes = layer_attn_bytes(wl)
    prefill = args.workload == "c3"
    if prefill:
        # the query-blocked indexer: bf16 MFMA over the causal rectangle
        flops = sum(2.0 * 32 * 128 * (p + 1) for p in wl.q_pos)
        tflops = flops / (kern_ms["indexer"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "indexer_prefill_kernel", "flops_per_launch": flops,
                    "avg_launch_ms": round(kern_ms["indexer"], 5)}
    else:
        idx_gbs = idx_bytes / (kern_ms["indexer"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(idx_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                    "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "kernel": "indexer_decode_kernel", "bytes_per_launch": idx_bytes,
                    "avg_launch_ms": round(kern_ms["indexer"], 5)}

    out = {
        "metric": "sparse-attn decode queries/s + HBM GB/s at 128K ctx; indexer prefill TFLOP/s",
        "value": round(wl.n_q / (ms_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "n_q": wl.n_q, "layers": wl.n_layers,
                   "full_layers": sum(wl.full), "context_tokens": wl.total_tokens,
                   "topk": 2048, "heads": 64, "index_heads": 32, "seed": args.seed},
        # HBM rates describe the decode workloads; the prefill stack is MFMA-bound
        "hbm_gbs_step": None if prefill else round(total_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_bytes": None if prefill else total_bytes,
        "roofline": roofline,
        # the whole step against the HBM roofline: algorithmic bytes of one
        # step over the graph-replay time
        "step_roofline": None if prefill else {
            "bound": "hbm", "achieved": round(total_bytes / (ms_step * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_step": total_bytes, "ms_per_step": round(ms_step, 5)},
        "replay_ms": replay_ms,
        "kernel_ms_first_layer": {n: round(v, 5) for n, v in kern_ms.items()},
        # where an eager step's time goes: the indexer and top-k of the full
        # layer, and everything after them (attention + W_UV of all layers)
        "stage_fractions_eager": stage_fractions(kern_ms, eager_ms),
        "attn_layer_gbs": None if prefill else round(attn_bytes / (kern_ms["attn"] * 1e-3) / 1e9, 1),
        # query tokens x layers per second over the graph replays, and the
        # rate of one layer's attention stage alone (sa_mla_sparse_attn's
        # work: attention + merge + W_UV, from the first layer's events)
        "layer_queries_per_s": round(wl.n_q * wl.n_layers / (ms_step * 1e-3), 1),
        "attn_stage_queries_per_s": round(wl.n_q / (kern_ms["attn"] * 1e-3), 1),
        "eager_ms_per_step": round(eager_ms, 5),
        "input_copies": len(stacks),
        "env": environment(torch, sclk_after),
    }
    if not args.no_prefill:
        print("[bench] prefill indexer", file=sys.stderr, flush=True)
        out["prefill_indexer"] = prefill_indexer(args.seed)
        print("[bench] cache write", file=sys.stderr, flush=True)
        out["cache_write"] = cache_write_leg(args.seed)
    if not args.no_fp8 and not prefill:
        print("[bench] fp8 caches", file=sys.stderr, flush=True)
        out["decode_fp8"] = fp8_leg(batches, wl, args.steps, args.warmup)
    if not args.no_query:
        print("[bench] query side", file=sys.stderr, flush=True)
        out["query_side"] = {"decode_16_tokens": query_side_leg(args.seed, 16),
                             "prefill_4096_tokens": query_side_leg(args.seed, 4096)}
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(b, wl, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
