#!/usr/bin/env python3
"""Benchmark of the paged decode path on one MI355X.

Default workload: one Llama-3-8B-shaped attention layer at decode time — batch 32,
32 query / 8 kv heads (GQA 4), head_dim 128, bf16 cache, 16-token blocks, context
lengths drawn uniformly from [1024, 4096], random block tables. One step is the whole
hot path over one batch: paged_decode_append_attention, i.e. the append of the 32 new
tokens fused into the persistent split-K attention kernel, then the log-sum-exp combine.
Several replica caches (own pools, tables, queries) are cycled so that consecutive steps
never find their K/V in the 256 MB last-level cache; every replica has the same context
lengths, so the bytes per step are fixed.

Prints one JSON line. value = algorithmic KV bytes per step (the attended tokens' K and V
rows, sum(L) * 2 * Hkv * d * 2 bytes) / wall time per step, over the timed steps, which run
with no event records at all. roofline = the main attention kernel alone: the same bytes /
its mean duration, from HIP events the library records on its launch stream around the
kernel, in a separate loop of at least 50 launches after the timed region. cpu_baseline =
the oracle timed on the host (one thread, and one GPU's share of host threads).

--workload selects one of the other four workloads (report lines with the same fields).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode-attention KV GB/s and % of HBM peak; decode steps/s per layer"
HBM_PEAK_GBS = 8000.0
ORACLE_THREADS = 16  # host threads of one GPU's share of the box (at most nproc)
MIN_EVENT_LAUNCHES = 50

# The sources that define the measured kernels and their launch (grid, split plan): a change to
# any of them invalidates the committed HBM counters.
KERNEL_SOURCES = ("api.hip", "append.hip", "decode.hip", "pkv_device.h", "pkv_internal.h", "pkv_plan.h", "pkv_q8.h",
                  "stream.hip")


def code_only(text: str) -> str:
    """C/C++/HIP source without its comments, trailing blanks and empty lines (the sources carry no
    comment markers inside string literals)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(csrc: str = None) -> str:
    """sha256 over KERNEL_SOURCES (names and code without comments, in that order): an edit to a
    comment keeps the committed counters valid, any edit to the code does not."""
    import hashlib
    csrc = csrc or os.path.join(ROOT, "paged_kv_cache_16_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 --pmc record
    (profiles/<kernel>_<workload>_traffic.json), or None when none matches the current kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return int(round(rec["traffic_bytes"]))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama3_8b_layer_bf16")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--split-tokens", type=int, default=0, help="0 = the library's automatic plan")
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU baseline: oracle time to spend single-threaded on a sample of the workload "
                         "(0 = skip)")
    ap.add_argument("--event-launches", type=int, default=100,
                    help="launches of the separate event-timed loop after the timed region (at least 50)")
    ap.add_argument("--no-graph", action="store_true", help="multi-layer modes: skip the HIP-graph timing")
    ap.add_argument("--scores", action="store_true",
                    help="default workload: every step also exports the decode-time KV scores "
                         "(softmax probability per token and kv head, accumulated over steps)")
    ap.add_argument("--kv-dtype", default=None, choices=[None, "int8"],
                    help="default workload: keep the cache in INT8 (per-row scales); bytes count the int8 "
                         "data plus the scales actually read")
    ap.add_argument("--loop", action="store_true",
                    help="page-selected workload: close the loop; each step exports per-page scores and "
                         "paged_select_pages picks the next step's pages from them (newest page kept)")
    ap.add_argument("--policy", action="store_true",
                    help="multi-layer workloads with window layers: per-layer memory policy; window layers keep "
                         "only sink pages plus a ring of pages in pools of their own, and every layer's table "
                         "and slots come from the library's block manager")
    ap.add_argument("--context", type=int, default=0,
                    help="default workload: every sequence at this context length instead of U[1024, 4096] "
                         "(4001: the 4000-token prompt plus one decode step)")
    ap.add_argument("--tp-share", type=int, default=1,
                    help="default workload at one tensor-parallel GPU's share: kv and query heads divided by "
                         "this (8: 1 kv head, 4 query heads); 16 replicas so the MALL cannot serve repeats")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    ap.add_argument("--read-probe-mib", type=int, default=2048,
                    help="after the timed region, time the library's read-rate probe over this many MiB "
                         "(0: skip); the roofline then also gives achieved / probe")
    ap.add_argument("--noalloc", action="store_true",
                    help="default workload: time paged_decode_attention_noalloc (append + attention through "
                         "the library's scratch) instead of the fused step")
    return ap.parse_args()


def read_probe_gbs(mib: int, dev) -> dict:
    """Best rate of pkv_read_probe (16-byte nontemporal loads, every wave on its own contiguous
    share) over a buffer far larger than the last-level cache, at 1, 2 and 4 waves per SIMD."""
    import torch
    import paged_kv_cache_16_amd as pkv
    buf = torch.zeros(mib << 20, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(cus * 4 * 4, dtype=torch.int32, device=dev)
    best = (0.0, 0)
    for wps in (1, 2, 4):
        nbytes = 0
        for _ in range(3):
            nbytes = pkv.read_probe(buf, wps, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            pkv.read_probe(buf, wps, sink)
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        best = max(best, (gbs, wps))
    del buf, sink
    return {"gbs": round(best[0], 1), "waves_per_simd": best[1], "mib": mib}


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its launch stream)."""

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev: int, stream: int) -> None:
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self) -> int:
        h = self._ct.c_void_p()
        if self.lib.hipEventCreate(self._ct.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self._ct.c_float()
        if self.lib.hipEventElapsedTime(self._ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, h: int) -> None:
        self.lib.hipEventDestroy(h)


def host_info() -> dict:
    """The host's logical CPU count and CPU model, as this process sees them."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def event_loop(call, n: int, hip) -> list:
    """Runs call(timing) n times, each launch with its own event pair that the library records
    on its launch stream right around the main attention kernel; returns the durations (ms),
    sorted."""
    import torch
    evs = [(hip.create(), hip.create()) for _ in range(n)]
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    ms = sorted(hip.elapsed_ms(a, b) for a, b in evs)
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return ms


def roofline(kernel: str, bytes_per_launch: int, ms: list, traffic, probe) -> dict:
    """The roofline object of one kernel: algorithmic bytes per launch / mean event duration."""
    mean = statistics.fmean(ms)
    q = lambda f: ms[min(len(ms) - 1, int(f * len(ms)))]
    achieved = bytes_per_launch / (mean * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_unit": "bytes per launch",
         "bytes_per_launch": bytes_per_launch, "mean_us": round(mean * 1e3, 3), "p10_us": round(q(0.1) * 1e3, 3),
         "p50_us": round(q(0.5) * 1e3, 3), "p90_us": round(q(0.9) * 1e3, 3), "samples": len(ms),
         "timing": "separate loop after the timed region, one event pair per launch"}
    if probe:
        r.update(read_probe_gbs=probe["gbs"], frac_of_read_probe=round(achieved / probe["gbs"], 4), read_probe=probe)
    return r


def build_replica(w, lens, seed, r, dev, kv_dtype=None):
    """One replica of the workload's caches and step inputs. kv_dtype "int8": an INT8 cache
    filled by the quantising append from the same rows."""
    import torch

    import paged_kv_cache_16_amd as pkv
    import synth

    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    tdt = synth.TORCH_DTYPE[w.dtype]
    bt, nb = synth.block_tables(lens, P, seed, w.name, r)
    gk = pkv.new_cache(nb, Hkv, P, d, torch.int8 if kv_dtype == "int8" else tdt, device=dev)
    gv = torch.empty_like(gk)
    for b, L in enumerate(lens):  # prefill: tokens [0, L-1) of every sequence
        if L > 1:
            kb = synth.normal((L - 1, Hkv, d), seed, w.name, r, b, "k", dtype=w.dtype, device=dev)
            vb = synth.normal((L - 1, Hkv, d), seed, w.name, r, b, "v", dtype=w.dtype, device=dev)
            sl = synth.token_slots(bt[b:b + 1], [L - 1], P).to(dev)
            pkv.kv_cache_append(gk, gv, kb, vb, sl)
    rep = dict(
        k=gk, v=gv, bt=bt.to(dev),
        cl=torch.tensor(lens, dtype=torch.int32, device=dev),
        q=synth.normal((B, Hq, d), seed, w.name, r, "q", dtype=w.dtype, device=dev),
        k_new=synth.normal((B, Hkv, d), seed, w.name, r, "knew", dtype=w.dtype, device=dev),
        v_new=synth.normal((B, Hkv, d), seed, w.name, r, "vnew", dtype=w.dtype, device=dev),
        slots=torch.tensor([synth.slot_of(bt, b, L - 1, P) for b, L in enumerate(lens)],
                           dtype=torch.int32, device=dev),
        bt_cpu=bt,
    )
    return rep


# ---------------------------------------------------------------------------------- CPU baseline
# The oracle as it stands (plain fp64 C), timed on the host on a bounded sample of the same
# workload: single-threaded, then the same sample as one oracle call per sequence on a pool of
# host threads (the C oracle runs outside the interpreter lock). Only the attention calls are
# timed; building the oracle's pools is not.
def _oracle_seq(dtype, K_rows, V_rows, n_tokens, P, Hkv, d, seed, tokens=None):
    """An oracle pool holding one sequence's rows (of `tokens`, default 0 .. m-1), under a
    seeded table. Returns (kpool, vpool, block_table [1, pages])."""
    import numpy as np
    import synth
    import oracle
    bt, nb = synth.block_tables([n_tokens], P, seed, "cpu-baseline")
    raw_t = np.float32 if dtype == "f32" else np.uint16
    kp = np.zeros(nb * Hkv * P * d, raw_t)
    vp = np.zeros_like(kp)
    t = np.arange(K_rows.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    slots = (bt[0].numpy().astype(np.int64)[t // P] * P + t % P).astype(np.int32)
    oracle.kv_append(dtype, kp, vp, synth.raw_numpy(K_rows), synth.raw_numpy(V_rows), slots, P=P, Hkv=Hkv, d=d)
    return kp, vp, bt.numpy()


def _time_calls(builders, budget_s):
    """builders: callables that prepare one oracle call (untimed) and return it. Prepares and
    times the calls one by one until budget_s is spent (at least one); then runs the same calls on
    the thread pool, timed as a whole. Returns (n_done, single_s, parallel_s, threads)."""
    from concurrent.futures import ThreadPoolExecutor
    fns, single = [], 0.0
    for build in builders:
        if fns and single >= budget_s:
            break
        fn = build()
        t0 = time.perf_counter()
        fn()
        single += time.perf_counter() - t0
        fns.append(fn)
    threads = max(1, min(ORACLE_THREADS, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda f: f(), fns))
        par = time.perf_counter() - t0
    return len(fns), single, par, threads


def cpu_baseline(w, args, dev, lens=None):
    """The oracle's time on a bounded sample of workload w, scaled to the workload's own unit:
    per attention call (one layer of the batch) for single-layer workloads, per layer-step and
    per decode step for multi-layer ones. value = algorithmic K/V bytes / oracle seconds (GB/s,
    one thread)."""
    import numpy as np
    import torch

    import oracle
    import synth

    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    seed, budget = args.seed, args.cpu_seconds
    bpt = w.kv_bytes_per_token()
    if lens is None:
        lens = [w.ctx_lo] * B if w.ctx_lo == w.ctx_hi else \
            synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, seed, w.name).tolist()
    if w.steps > 1:
        lens = [L + 1 for L in lens]  # the first decode step (cached context plus the new token)

    def rows(b, tag, n):
        return synth.normal((n, Hkv, d), seed, w.name, "cpu", b, tag, dtype=w.dtype, device=dev).cpu()

    def seq_call(b, L, okw=None, tokens=None):
        """A timed closure: the oracle's attention over sequence b (its pool built now)."""
        okw = okw or {}
        n = len(tokens) if tokens is not None else L
        idx = None if tokens is None else torch.as_tensor(tokens)
        K, V = rows(b, "k", L), rows(b, "v", L)
        if idx is not None:
            K, V = K[idx], V[idx]
        kp, vp, bt = _oracle_seq(w.dtype, K, V, L, P, Hkv, d, seed, tokens)
        q = synth.raw_numpy(synth.normal((1, Hq, d), seed, w.name, "cpu", b, "q", dtype=w.dtype))
        cl = np.array([L], np.int32)
        assert n == K.shape[0]
        return lambda: oracle.decode_attention(w.dtype, kp, vp, q, bt, cl, P=P, Hkv=Hkv, d=d, **okw)

    info = host_info()
    res = {"unit": "GB/s", "kind": "oracle", **info}
    if w.pages_per_step:  # whole calls: every sequence over its page list
        pl = synth.page_lists(lens, P, w.pages_per_step, seed, w.name, "cpu").numpy()
        calls = []
        for b, L in enumerate(lens):
            toks = np.concatenate([np.arange(p * P, min((p + 1) * P, L)) for p in pl[b] if p >= 0])
            calls.append(seq_call(b, L, dict(page_list=pl[b:b + 1]), toks))
        call_bytes = B * w.pages_per_step * P * bpt
        reps = []
        t_single = 0.0
        while not reps or t_single < budget:
            t0 = time.perf_counter()
            for fn in calls:
                fn()
            reps.append(time.perf_counter() - t0)
            t_single += reps[-1]
        _, _, par, threads = _time_calls([lambda fn=fn: fn for fn in calls], 0.0)
        per_call = statistics.fmean(reps)
        res.update(value=round(call_bytes / per_call / 1e9, 4), cores=1, seconds_per_call=round(per_call, 4),
                   sample=f"{len(reps)} whole calls ({B} sequences x {w.pages_per_step} pages of {P} tokens, "
                          f"all {Hq} heads), single-threaded fp64 C oracle, {t_single:.2f} s",
                   parallel={"value": round(call_bytes / par / 1e9, 4), "unit": "GB/s", "cores": threads,
                             "seconds_per_call": round(par, 4),
                             "sample": f"one whole call, one oracle call per sequence on {threads} host threads"})
        return res
    if w.name == "tiny_mha_f32":  # whole calls
        fn = seq_call(0, lens[0])
        reps, t_single = [], 0.0
        while not reps or t_single < min(budget, 2.0):
            t0 = time.perf_counter()
            fn()
            reps.append(time.perf_counter() - t0)
            t_single += reps[-1]
        per_call = statistics.fmean(reps)
        call_bytes = sum(lens) * bpt
        res.update(value=round(call_bytes / per_call / 1e9, 4), cores=1, seconds_per_call=round(per_call, 6),
                   sample=f"{len(reps)} whole calls (1 sequence of {lens[0]} tokens, {Hq} heads), "
                          f"single-threaded fp64 C oracle, {t_single:.2f} s")
        return res
    # sequences of the workload (full attention), sampled in order until the budget is spent
    builders = [lambda b=b, L=L: seq_call(b, L) for b, L in enumerate(lens)]
    seq_bytes = [L * bpt for L in lens]
    done, single, par, threads = _time_calls(builders, budget if not w.window_layers else budget / 2)
    sb = sum(seq_bytes[:done])
    rate1, rate_p = sb / single, sb / par
    full_call = sum(lens) * bpt  # one full layer of the batch
    res.update(value=round(rate1 / 1e9, 4), cores=1,
               sample=f"{done} whole sequences ({sum(lens[:done])} tokens, all {Hq} query heads, full attention) "
                      f"of the workload, one oracle call each, single-threaded fp64 C oracle, {single:.2f} s; "
                      f"per-call figures scale this rate to the whole batch",
               parallel={"value": round(rate_p / 1e9, 4), "unit": "GB/s", "cores": threads, "seconds": round(par, 3),
                         "sample": f"the same sequences, one oracle call per sequence on {threads} host threads, "
                                   f"timed as a whole"})
    if w.layers == 1:
        res["seconds_per_call"] = round(full_call / rate1, 4)
        res["parallel"]["seconds_per_call"] = round(full_call / rate_p, 4)
        return res
    n_full = w.layers - len(w.window_layers)
    per_full = full_call / rate1
    res["seconds_per_layer_step"] = round(per_full, 4) if not w.window_layers else None
    if w.window_layers:  # window layer-steps timed whole: every sequence, window + sinks
        wcalls = []
        for b, L in enumerate(lens):
            toks = np.concatenate([np.arange(min(w.sinks, L)), np.arange(max(min(w.sinks, L), L - w.window), L)])
            wcalls.append(seq_call(b, L, dict(window=w.window, sinks=w.sinks), toks))
        t0 = time.perf_counter()
        for fn in wcalls:
            fn()
        per_win = time.perf_counter() - t0
        res["seconds_per_full_layer_step"] = round(per_full, 4)
        res["seconds_per_window_layer_step"] = round(per_win, 4)
        res["seconds_per_step"] = round(n_full * per_full + len(w.window_layers) * per_win, 3)
        res["sample"] += (f"; window layer-step: the {B} window calls (window {w.window} + {w.sinks} sinks) "
                          f"timed whole")
    else:
        res["seconds_per_step"] = round(w.layers * per_full, 3)
        res["sample"] += f"; lengths at the first decode step ({min(lens)}..{max(lens)})"
    return res


def _layer_caches(w, lens, P, seed, dev, tag, bt, nb=None, slots=None):
    """One layer's K/V pools, prefilled with tokens [0, L_b - 1) of every sequence: at the slots
    of the plain table bt, or at slots[b] (the block manager's, for a pool of nb blocks)."""
    import torch

    import paged_kv_cache_16_amd as pkv
    import synth

    d, Hkv = w.head_dim, w.kv_heads
    nb = int(bt.max()) + 1 if nb is None else nb
    gk = torch.empty((nb, Hkv, P, d), dtype=synth.TORCH_DTYPE[w.dtype], device=dev)
    gv = torch.empty_like(gk)
    for b, L in enumerate(lens):
        if L > 1:
            kb = synth.normal((L - 1, Hkv, d), seed, w.name, tag, b, "k", dtype=w.dtype, device=dev)
            vb = synth.normal((L - 1, Hkv, d), seed, w.name, tag, b, "v", dtype=w.dtype, device=dev)
            sl = synth.token_slots(bt[b:b + 1], [L - 1], P).to(dev) if slots is None else slots[b]
            pkv.kv_cache_append(gk, gv, kb, vb, sl)
    return gk, gv


def _policy_setup(w, base, steps, P, bt, nb, dev):
    """Per-layer memory policy: group 0 = full layers (nb blocks), group 1 = window layers (a
    ring of sink pages + R pages per sequence). The block manager takes the prefill of L-1
    tokens and then every step's new tokens; returns its slots and tables on the device."""
    import numpy as np
    import torch

    import paged_kv_cache_16_amd as pkv

    B = len(base)
    R = pkv.ring_pages(w.window, P)
    nb_ring = B * (-(-w.sinks // P) + R)
    bm = pkv.BlockManager(P, B, bt.shape[1], [dict(num_blocks=nb), dict(window=w.window, num_sinks=w.sinks,
                                                                       num_blocks=nb_ring)])
    ids = np.arange(B, dtype=np.int32)
    pre, _ = bm.append(ids, [L - 1 for L in base])
    pre_slots = []
    for g in range(2):
        cuts = np.cumsum([0] + [L - 1 for L in base])
        pre_slots.append([torch.from_numpy(pre[g, cuts[b]:cuts[b + 1]].copy()).to(dev) for b in range(B)])
    step_slots = []
    for _ in range(steps):
        sl, _ = bm.append(ids)
        step_slots.append([torch.from_numpy(sl[g].copy()).to(dev) for g in range(2)])
    # tables only gain entries after a page is first reached, so the last step's tables serve
    # every step
    tables = [torch.from_numpy(bm.block_table(g, ids)).to(dev) for g in range(2)]
    in_use = [bm.blocks_in_use(g) for g in range(2)]
    # host cost of the manager per decode step (through the Python binding): one append for the
    # batch and both tables
    n = 2000
    bm2 = pkv.BlockManager(P, B, bt.shape[1] + n // P + 1, [dict(num_blocks=nb + B * (n // P + 1)),
                                               dict(window=w.window, num_sinks=w.sinks, num_blocks=nb_ring)])
    bm2.append(ids, [L - 1 for L in base])
    t0 = time.perf_counter()
    for _ in range(n):
        bm2.append(ids)
        bm2.block_table(0, ids)
        bm2.block_table(1, ids)
    host_us = (time.perf_counter() - t0) * 1e6 / n
    bm.close()
    bm2.close()
    return dict(R=R, nb_ring=nb_ring, pre_slots=pre_slots, step_slots=step_slots, tables=tables, in_use=in_use,
                host_us=host_us)


def run_layer(w, args, dev):
    """Single-layer workloads (the default Llama-3-8B-shaped layer and its variants, and the
    tiny MHA check): one decode step of the layer per timed step."""
    import itertools

    import torch

    import paged_kv_cache_16_amd as pkv
    import synth

    variant = args.context > 0 or args.tp_share > 1
    if variant:
        if w.kv_heads % args.tp_share:
            print(f"bench.py: {w.kv_heads} kv heads do not split {args.tp_share} ways", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, kv_heads=w.kv_heads // args.tp_share, q_heads=w.q_heads // args.tp_share)
        if args.tp_share > 1 and args.replicas == 8:
            args.replicas = 16
    if args.context > 0:
        lens = [args.context] * w.batch
    elif w.ctx_lo == w.ctx_hi:
        lens = [w.ctx_lo] * w.batch
    else:
        lens = synth.uniform_lengths(w.batch, w.ctx_lo, w.ctx_hi, args.seed, w.name).tolist()
    kv_bytes = sum(lens) * w.kv_bytes_per_token()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Built last-first. The first step over the replica whose prefill ran last took ≈20 µs longer
    # than any other step (the step over replica 7 when 5 warmup steps cover replicas 0-4); built
    # in this order that replica is 0, which the first warmup step reads.
    reps = [None] * args.replicas
    for r in reversed(range(args.replicas)):
        reps[r] = build_replica(w, lens, args.seed, r, dev, args.kv_dtype)
    if args.kv_dtype == "int8":  # K and V: d int8 bytes + one fp32 scale per token and kv head
        kv_bytes = sum(lens) * 2 * w.kv_heads * (w.head_dim + 4)
    torch.cuda.synchronize()
    B, Hq, d = w.batch, w.q_heads, w.head_dim
    mcl = max(lens)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = pkv.workspace_size(reps[0]["k"], B, Hq, mcl, split_tokens=args.split_tokens, scores=args.scores)
    workspace = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    scores = torch.zeros((B, w.kv_heads, mcl), dtype=torch.float32, device=dev) if args.scores else None
    hip = HipEvents()

    # each replica's step checked and marshalled once: a timed step is one library call
    prepared = {id(rep): pkv.prepare_decode_append_attention(
        rep["q"], rep["k"], rep["v"], rep["k_new"], rep["v_new"], rep["slots"], rep["bt"], rep["cl"],
        max_context_len=mcl, split_tokens=args.split_tokens, out=out, lse=lse, workspace=workspace,
        scores=scores) for rep in reps}

    def step(rep, ev=None):
        if args.noalloc:  # the append, then attention over the library's own scratch
            pkv.kv_cache_append(rep["k"], rep["v"], rep["k_new"], rep["v_new"], rep["slots"])
            pkv.profile_events(*(ev or (None, None)))
            pkv.paged_decode_attention_noalloc(rep["q"], rep["k"], rep["v"], rep["bt"], rep["cl"],
                                               max_context_len=mcl, split_tokens=args.split_tokens, out=out,
                                               lse=lse, scores=scores)
            pkv.profile_events()
            return
        # one decode step of the layer: append of the 32 new tokens + attention, fused
        if ev is not None:
            pkv.profile_events(*ev)
        prepared[id(rep)]()
        if ev is not None:
            pkv.profile_events()

    for i in range(args.warmup):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9

    # the main kernel alone: a separate loop, one event pair per launch, replicas cycled on
    ctr = itertools.count(args.steps)
    kern_ms = event_loop(lambda ev: step(reps[next(ctr) % len(reps)], ev),
                         max(MIN_EVENT_LAUNCHES, args.event_launches), hip)
    probe = read_probe_gbs(args.read_probe_mib, dev) if args.read_probe_mib > 0 else None

    dt = {"bf16": "BF16", "f16": "F16", "f32": "F32"}[w.dtype]
    if args.kv_dtype == "int8":
        kname = f"decode_stream_kernel<I8B,{d},full" + (">" if args.noalloc else ",fused append>")
    elif args.split_tokens:
        kname = f"decode_split_kernel<{dt},{d},full>"
    elif ws_bytes == 0:  # short sequences: the one-kernel path
        kname = f"decode_split_kernel<{dt},{d},full,one kernel" + (">" if args.noalloc else ",fused append>")
    else:
        kname = f"decode_stream_kernel<{dt},{d},full" + (">" if args.noalloc else ",fused append>")
    plain = not (args.scores or variant or args.split_tokens or args.noalloc)
    step_desc = ("paged_decode_append_attention: append of the new tokens fused into the persistent split "
                 "kernel, then the LSE combine")
    if args.kv_dtype == "int8":
        step_desc = ("paged_decode_append_attention on an INT8 cache: the new tokens quantised inside the "
                     "persistent split kernel, then the LSE combine, which stores the quantised rows")
    if args.noalloc:
        step_desc = "kv_cache_append, then paged_decode_attention_noalloc (workspace in the library's scratch)"
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "cache_dtype": args.kv_dtype or w.dtype,
            "context": (f"all {lens[0]}" if len(set(lens)) == 1 else f"U[{w.ctx_lo},{w.ctx_hi}] seed {args.seed}")
            + f", sum {sum(lens)}, max {mcl}",
            "tp_share": args.tp_share,
            "replicas": args.replicas, "split_tokens": args.split_tokens,
            "step": step_desc + (", plus the decode-time KV score export" if args.scores else ""),
            "kv_dtype": args.kv_dtype or w.dtype,
            "parallelism": "single GPU",
        },
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "steps_per_s_per_layer": round(1e3 / ms_per_step, 1),
        "kv_bytes_per_step": kv_bytes,
        "roofline": roofline(kname, kv_bytes, kern_ms,
                             measured_traffic(kname.split("<")[0], w.name + ("_int8" if args.kv_dtype else ""))
                             if plain else None, probe),
    }
    return res, lens, variant


def run_multilayer(w, args, dev):
    """Decode steps over all layers: per layer, append of the batch's new tokens and attention
    (window + sinks on the window layers); the context advances once per step after the last
    layer. Qwen2.5-1.5B shape: 4096 cached tokens, then 32 steps (L = 4097..4128). KV-sparse
    Llama-3-8B shape: one step, repeated for timing."""
    import torch

    import paged_kv_cache_16_amd as pkv
    import synth

    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    if w.ctx_lo == w.ctx_hi:
        base = [w.ctx_lo + 1] * B  # L at the first step
    else:
        base = synth.uniform_lengths(B, w.ctx_lo, w.ctx_hi, args.seed, w.name).tolist()
    steps = w.steps
    cap = [L + steps - 1 for L in base]
    bt, nb = synth.block_tables(cap, P, args.seed, w.name)
    gbt = bt.to(dev)
    policy = _policy_setup(w, base, steps, P, bt, nb, dev) if args.policy and w.window_layers else None
    slots_plain = [torch.tensor([synth.slot_of(bt, b, L + s - 1, P) for b, L in enumerate(base)],
                                dtype=torch.int32, device=dev) for s in range(steps)]
    layers = []
    for layer in range(w.layers):
        win = layer in w.window_layers
        if policy:
            g = 1 if win else 0
            gk, gv = _layer_caches(w, base, P, args.seed, dev, 1000 + layer, bt,
                                   nb=policy["nb_ring"] if win else nb, slots=policy["pre_slots"][g])
            table, slots, ring = policy["tables"][g], [st[g] for st in policy["step_slots"]], policy["R"] if win else 0
        else:
            gk, gv = _layer_caches(w, base, P, args.seed, dev, 1000 + layer, bt)
            table, slots, ring = gbt, slots_plain, 0
        layers.append(dict(
            k=gk, v=gv, bt=table, slots=slots, ring=ring,
            q=synth.normal((B, Hq, d), args.seed, w.name, layer, "q", dtype=w.dtype, device=dev),
            kn=synth.normal((steps, B, Hkv, d), args.seed, w.name, layer, "kn", dtype=w.dtype, device=dev),
            vn=synth.normal((steps, B, Hkv, d), args.seed, w.name, layer, "vn", dtype=w.dtype, device=dev),
            window=w.window if win else 0))
    lens_s = [torch.tensor([L + s for L in base], dtype=torch.int32, device=dev) for s in range(steps)]
    mcl = max(cap)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(256, max(pkv.workspace_size(layers[0]["k"], B, Hq, mcl, window=ly["window"],
                                                     num_sinks=w.sinks) for ly in layers)),
                     dtype=torch.uint8, device=dev)
    hip = HipEvents()

    # every (step, layer) call checked and marshalled once: a timed layer-step is one library call
    prepared = [[pkv.prepare_decode_append_attention(
        ly["q"], ly["k"], ly["v"], ly["kn"][s], ly["vn"][s], ly["slots"][s], ly["bt"], lens_s[s],
        max_context_len=mcl, window=ly["window"], num_sinks=w.sinks if ly["window"] else 0, out=out, lse=lse,
        workspace=ws, ring_pages=ly["ring"]) for ly in layers] for s in range(steps)]

    def step(s, layer_timing=None):
        for li, call in enumerate(prepared[s]):
            if layer_timing:
                pkv.profile_events(*layer_timing(li))
            call()
        if layer_timing:
            pkv.profile_events()

    reps = max(1, args.steps // (w.layers * steps)) if steps > 1 else max(4, args.steps // 8)
    for s in range(min(steps, 4)):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        for s in range(steps):
            step(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    n_steps = reps * steps
    bytes_total = 0
    for s_i in range(n_steps):
        s = s_i % steps
        for ly in layers:
            if ly["window"]:
                att = sum(min(L + s, ly["window"] + min(w.sinks, L + s)) for L in base)
            else:
                att = sum(L + s for L in base)
            bytes_total += att * w.kv_bytes_per_token()

    # the kernels alone: a separate loop of whole steps, every layer's main kernel between its
    # own event pair (steps cycled from the first)
    ev_steps = max(1, -(-MIN_EVENT_LAUNCHES // max(1, w.layers - len(w.window_layers))))
    ev_steps = max(ev_steps, min(steps, 4))
    evs = [[(hip.create(), hip.create()) for _ in layers] for _ in range(ev_steps)]
    for i in range(ev_steps):
        step(i % steps, layer_timing=lambda li, i=i: evs[i][li])
    torch.cuda.synchronize()
    full_s, win_s = [], []  # (bytes, ms) per launch
    for i in range(ev_steps):
        s = i % steps
        for li, ly in enumerate(layers):
            ms = hip.elapsed_ms(*evs[i][li])
            if ly["window"]:
                att = sum(min(L + s, ly["window"] + min(w.sinks, L + s)) for L in base)
                win_s.append((att * w.kv_bytes_per_token(), ms))
            else:
                full_s.append((sum(L + s for L in base) * w.kv_bytes_per_token(), ms))
            hip.destroy(evs[i][li][0])
            hip.destroy(evs[i][li][1])
    full_us = [m * 1e3 for _, m in full_s]
    win_us = [m * 1e3 for _, m in win_s]
    step_ms = elapsed * 1e3 / n_steps
    graph_ms = None
    if not args.no_graph:
        # The same steps replayed from HIP graphs: one graph per decode step holding every layer.
        # (captured through the plain wrapper: a prepared call is bound to the stream current when
        # it was prepared, and capture runs on a stream of its own)
        def step_on_current_stream(s):
            for ly in layers:
                pkv.paged_decode_append_attention(ly["q"], ly["k"], ly["v"], ly["kn"][s], ly["vn"][s],
                                                  ly["slots"][s], ly["bt"], lens_s[s], max_context_len=mcl,
                                                  window=ly["window"], num_sinks=w.sinks if ly["window"] else 0,
                                                  out=out, lse=lse, workspace=ws, ring_pages=ly["ring"])

        graphs = []
        for s in range(steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_on_current_stream(s)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs[:4]:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / n_steps
        del graphs
    res = {
        "metric": METRIC, "value": round(bytes_total / elapsed / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": n_steps, "warmup": min(steps, 4), "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "block_size": P, "layers": w.layers, "decode_steps": steps,
                   "context_at_first_step": f"{min(base)}..{max(base)}",
                   "window_layers": len(w.window_layers), "window": w.window, "sinks": w.sinks,
                   "step": "per layer: paged_decode_append_attention (append fused into attention)",
                   "parallelism": "single GPU"},
        "full_steps_per_s": round(1e3 / step_ms, 2),
        "layer_steps_per_s": round(1e3 / step_ms * w.layers, 1),
        "graph_full_steps_per_s": round(1e3 / graph_ms, 2) if graph_ms else None,
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms else None,
        "attention_us_full_layer_mean": round(statistics.fmean(full_us), 2) if full_us else None,
        "attention_us_window_layer_mean": round(statistics.fmean(win_us), 2) if win_us else None,
        "hbm_frac_of_peak": round(bytes_total / elapsed / 1e9 / HBM_PEAK_GBS, 4),
    }
    dt = {"bf16": "BF16", "f16": "F16", "f32": "F32"}[w.dtype]
    if full_s:
        res["roofline"] = roofline(f"decode_stream_kernel<{dt},{d},full,fused append>",
                                   int(statistics.fmean(b for b, _ in full_s)), sorted(m for _, m in full_s),
                                   None if policy else measured_traffic("decode_stream_kernel", w.name), None)
        res["roofline"]["note"] = "full layers; bytes_per_launch is the mean over the sampled steps"
    if win_s:
        res["roofline_window_layer"] = roofline(
            f"decode_split_kernel<{dt},{d},window,one kernel,fused append>",
            int(statistics.fmean(b for b, _ in win_s)), sorted(m for _, m in win_s),
            None if policy else measured_traffic("decode_split_kernel", w.name + "_window"), None)
    blk_bytes = 2 * Hkv * P * d * synth.DTYPE_BYTES[w.dtype]  # K and V of one block
    n_win = len(w.window_layers)
    res["kv_pool_bytes"] = w.layers * nb * blk_bytes
    if policy:
        res["config"]["memory_policy"] = (f"full layers: one block per page; window layers: ring of "
                                          f"{-(-w.sinks // P)} sink + {policy['R']} pages per sequence")
        res["kv_pool_bytes_policy"] = ((w.layers - n_win) * nb + n_win * policy["nb_ring"]) * blk_bytes
        # what the sequences hold at the last step, per the accounting of the [primer] KV formula
        res["kv_bytes_held"] = {
            "full_layers": (w.layers - n_win) * policy["in_use"][0] * blk_bytes,
            "window_layers": n_win * policy["in_use"][1] * blk_bytes,
            "all_layers_full_cache": w.layers * sum(pkv.kv_cache_bytes(1, 1, Hkv, d, L + steps - 1,
                                                                       synth.DTYPE_BYTES[w.dtype], P)
                                                    for L in base)}
        res["block_manager_us_per_step"] = round(policy["host_us"], 2)
    if full_us:
        per_layer_bytes = sum(base) * w.kv_bytes_per_token()  # first step's full-layer bytes
        res["attention_full_layer_GBps_at_step1"] = round(per_layer_bytes / (min(full_us) * 1e3), 1)
    return res


def run_page_selected(w, args, dev):
    """Page-selected decode: every step appends the new token and attends to 16 pages of each
    sequence (the newest page plus 15 distinct earlier ones), a fresh list per step."""
    import torch

    import paged_kv_cache_16_amd as pkv
    import synth

    B, P, d, Hkv, Hq = w.batch, w.block_size, w.head_dim, w.kv_heads, w.q_heads
    lens = [w.ctx_lo] * B
    bt, nb = synth.block_tables(lens, P, args.seed, w.name)
    gk, gv = _layer_caches(w, lens, P, args.seed, dev, "pages", bt)
    n_lists = 64
    lists = [synth.page_lists(lens, P, w.pages_per_step, args.seed, w.name, i).to(dev) for i in range(n_lists)]
    q = synth.normal((B, Hq, d), args.seed, w.name, "q", dtype=w.dtype, device=dev)
    kn = synth.normal((B, Hkv, d), args.seed, w.name, "kn", dtype=w.dtype, device=dev)
    vn = synth.normal((B, Hkv, d), args.seed, w.name, "vn", dtype=w.dtype, device=dev)
    slots = torch.tensor([synth.slot_of(bt, b, L - 1, P) for b, L in enumerate(lens)], dtype=torch.int32,
                         device=dev)
    cl = torch.tensor(lens, dtype=torch.int32, device=dev)
    gbt = bt.to(dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(256, pkv.workspace_size(gk, B, Hq, max(lens), page_list=lists[0])),
                     dtype=torch.uint8, device=dev)
    hip = HipEvents()

    loop = args.loop
    if loop:
        # closed loop: per-page scores accumulate over steps and pick the next step's pages
        n_pages = (max(lens) + P - 1) // P
        gscores = torch.zeros((B, Hkv, n_pages), dtype=torch.float32, device=dev)
        plist = lists[0].clone()
        ws = torch.zeros(max(256, pkv.workspace_size(gk, B, Hq, max(lens), page_list=lists[0], scores=True)),
                         dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    # each list's step (the loop's one step) checked and marshalled once
    if not loop:
        prepared = [pkv.prepare_decode_append_attention(q, gk, gv, kn, vn, slots, gbt, cl, max_context_len=max(lens),
                                                        page_list=lst, out=out, lse=lse, workspace=ws) for lst in lists]
    else:
        prepared = [pkv.prepare_decode_append_attention(q, gk, gv, kn, vn, slots, gbt, cl, max_context_len=max(lens),
                                                        page_list=plist, out=out, lse=lse, workspace=ws,
                                                        scores=gscores, score_block=P)]

    def step(i, ev=None, sev=None):
        if ev is not None:
            pkv.profile_events(*ev)
        prepared[i % len(prepared)]()
        if ev is not None:
            pkv.profile_events()
        if not loop:
            return
        if sev is not None:
            hip.record(sev[0], stream)
        pkv.select_pages(gscores, cl, block_size=P, k=w.pages_per_step, recent=1, page_list=plist)
        if sev is not None:
            hip.record(sev[1], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the kernels alone: a separate loop, one event pair per launch
    n_ev = max(MIN_EVENT_LAUNCHES, args.event_launches)
    evs = [(hip.create(), hip.create()) for _ in range(n_ev)]
    sevs = [(hip.create(), hip.create()) for _ in range(n_ev)] if loop else None
    for i in range(n_ev):
        step(i, evs[i], sevs[i] if loop else None)
    torch.cuda.synchronize()
    kern = sorted(hip.elapsed_ms(a, b) for a, b in evs)
    sel = sorted(hip.elapsed_ms(a, b) for a, b in sevs) if loop else []
    for a, b in evs + (sevs or []):
        hip.destroy(a)
        hip.destroy(b)
    att_bytes = B * w.pages_per_step * P * w.kv_bytes_per_token()
    step_ms = elapsed * 1e3 / args.steps
    kmean = statistics.fmean(kern)
    return {
        "metric": METRIC, "value": round(att_bytes / (step_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "block_size": P, "context": lens[0], "pages_per_step": w.pages_per_step,
                   "page_lists": n_lists, "pool_bytes": 2 * gk.numel() * gk.element_size(),
                   "step": "paged_decode_append_attention over the step's page list"
                           + (", per-page score export, paged_select_pages for the next step" if loop else ""),
                   "parallelism": "single GPU"},
        "hbm_frac_of_peak": round(att_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "steps_per_s_per_layer": round(1e3 / step_ms, 1),
        "attention_kernel_us_mean": round(kmean * 1e3, 3),
        "attention_kernel_GBps": round(att_bytes / (kmean * 1e-3) / 1e9, 2),
        **({"closed_loop": "per-page score export + paged_select_pages each step",
            "select_pages_us_mean": round(statistics.fmean(sel) * 1e3, 3),
            "select_pages_us_p50": round(sel[len(sel) // 2] * 1e3, 3)} if loop else {}),
        "roofline": roofline(f"decode_split_kernel<F16,{d},pages,one kernel,fused append"
                             + (",scores>" if loop else ">"), att_bytes, kern,
                             None if loop else measured_traffic("decode_split_kernel", w.name), None),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU; the decode path shards by kv head or by "
              "sequence with no exchange (see the design notes), and multi-GPU runs are not "
              "part of it. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_16_amd  # noqa: F401  (fails loudly when the library is not built)
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    lens, baseline_ok = None, True
    if w.layers > 1:
        res = run_multilayer(w, args, dev)
        baseline_ok = not args.policy
    elif w.pages_per_step:
        res = run_page_selected(w, args, dev)
        baseline_ok = not args.loop
    else:
        res, lens, variant = run_layer(w, args, dev)
        baseline_ok = not (args.kv_dtype or variant or args.scores or args.split_tokens or args.noalloc)
    if args.cpu_seconds > 0 and baseline_ok:
        res["cpu_baseline"] = cpu_baseline(w, args, dev, lens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
