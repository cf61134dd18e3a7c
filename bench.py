"""Benchmark of the MI355X DSA lightning indexer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-recall]
    python bench.py --copy-probe BYTES     (a plain device copy of known size, for calibrating
                                            the HBM byte counters of rocprofv3 --pmc)

One step = one full indexer call (every stage of the path: scoring, masking, top-k selection,
and for the variants the proxy / pooling / candidate stages) over one batch of seeded synthetic
input that is already resident in HBM. Prints ONE JSON line.

Without --workload the line is the metric's headline: the 64K prefill (dense64k) is the timed
step and its numbers are the line's value; the 128K decode step (decode128k) is timed after it
with the same steps and warmup and carried in the same line under "decode128k". With --workload
NAME the line is that workload alone; the group and block variants also report recall@k of their
selections against the dense indexer's GPU selection on the same inputs.

value = query-key pairs per second: the causally visible (query, key) pairs of the workload
(the work the dense indexer does; for the group and block variants this is the
dense-equivalent count) divided by the mean step time. Top-k rows per second are reported
beside it. roofline = the dominant kernel's algorithmic flops (or HBM bytes) per launch over its
mean launch duration, timed with HIP events recorded by the library on the launch stream.
cpu_baseline = the CPU oracle (float64 numpy) timed on a bounded row sample of the same
workload on this host. roofline.traffic = the dominant kernel's HBM bytes per launch from the
FETCH_SIZE / WRITE_SIZE counters recorded in profiles/traffic.json, each scaled by what the same
counter reads for a plain copy of known size; null when the kernel sources changed since.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer query-key pairs/sec + top-k rows/sec at 64K prefill, 128K decode; % roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# source files each profiled kernel is compiled from (its own file and the headers it includes)
KERNEL_SOURCES = {
    "score_kernel": ["score_kernel.h", "score_tile.h", "common.h", "kernels.h"],
    "decode_scan_kernel": ["decode.hip", "common.h", "kernels.h"],
    "block_refine_kernel": ["block_refine.hip", "score_tile.h", "common.h", "kernels.h"],
    "block_refine_direct_kernel": ["block_refine.hip", "score_tile.h", "common.h", "kernels.h"],
}


def csrc_digest(kernel):
    """sha256 over the sources of `kernel` and the build flags (changes whenever it may change)."""
    import hashlib
    pkg = os.path.join(ROOT, "sparse_attention_indexer_02_amd")
    h = hashlib.sha256()
    files = [os.path.join(pkg, "csrc", f) for f in KERNEL_SOURCES[kernel]]
    for f in files + [os.path.join(pkg, "build.py")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from profiles/traffic.json, or None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
        e = d["kernels"][f"{kernel}@{workload}"]
        if e["csrc_sha256"] != csrc_digest(kernel):
            return None
        c = d["copy"]
        rf = c["bytes"] / (c["fetch_kib"] * 1024.0)
        wf = c["bytes"] / (c["write_kib"] * 1024.0)
        return e["fetch_kib"] * 1024.0 * rf + e["write_kib"] * 1024.0 * wf
    except (OSError, KeyError, ValueError, ZeroDivisionError):
        return None


def block_refine_kernel_name(prob, block_size):
    """The refine kernel the library dispatches: bf16 queries and keys with a power-of-two block
    size, D of 64 or 128 and at most 64 heads stream the kept blocks straight into LDS."""
    import workloads as W
    direct = (prob.q_dtype == W.BF16 and prob.k_dtype == W.BF16 and block_size & (block_size - 1) == 0
              and prob.D in (64, 128) and prob.H <= 64)
    return "block_refine_direct_kernel" if direct else "block_refine_kernel"


def copy_probe(nbytes):
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": (nbytes // 4) * 4, "launches": 5}))


# ----------------------------------------------------------------------------------------------
# workloads: algorithmic work of the dominant kernel

def dense_flops(prob):
    """Score-contraction flops: 2 H Dk per visible pair, Dk the key row width (= D, or the latent
    width for absorbed queries)."""
    return 2.0 * prob.H * prob.k.shape[2] * prob.pairs()


def decode_bytes(prob):
    """Bytes the decode scan must read: every visible key row (+ its fp32 scale for FP8), the
    queries it scores with (the absorbed ones for a latent cache) and the head weights."""
    import numpy as np
    kl = prob.k_len.astype(np.int64)
    Dk = prob.k.shape[2]
    kb = Dk * (1 if prob.k_dtype == 2 else (2 if prob.k_dtype == 1 else 4))
    per_tok = kb + (4 if prob.k_dtype == 2 else 0)
    qbytes = prob.q.nbytes * Dk // prob.D
    return float((kl * per_tok).sum() + qbytes + prob.w.nbytes)


def group_refine_pairs(prob, G, C):
    """Pairs scored by the group path: proxy full-prefix scans + member refines over C."""
    import numpy as np
    T = prob.T
    NG = (T + G - 1) // G
    proxy = refine = 0
    for b in range(prob.B):
        pos = prob.q_pos[b].astype(np.int64)
        L = int(prob.k_len[b])
        top = [min(int(pos[g * G:min(T, (g + 1) * G)].max()) + 1, L) for g in range(NG)]
        proxy += sum(max(0, x) for x in top)
        refine += sum(min(C, max(0, top[g])) * (min(T, (g + 1) * G) - g * G) for g in range(NG))
    return proxy, refine


def given_pairs(prob, G, banks):
    """Pairs scored by the refine over given banks: each member's bank tokens inside its prefix."""
    import numpy as np
    n = 0
    for b in range(prob.B):
        for g in range(banks.shape[1]):
            v = np.unique(banks[b, g])
            v = v[v >= 0]
            for t in range(g * G, min(prob.T, g * G + G)):
                P = min(int(prob.q_pos[b, t]) + 1, int(prob.k_len[b]))
                n += int(np.searchsorted(v, P))
    return n


def gblock_refine_pairs(prob, G, Bs, keep):
    """Token pairs of the block-filtered proxy's member refine: min(keep, blocks eligible for the
    group's proxy) blocks of Bs tokens per member, cut to the member's prefix (the partial last
    block counted whole, as for the block path)."""
    import numpy as np
    n = 0
    for b in range(prob.B):
        pos = prob.q_pos[b].astype(np.int64)
        L = int(prob.k_len[b])
        NB = -(-L // Bs)
        for g in range((prob.T + G - 1) // G):
            mem = pos[g * G:min(prob.T, g * G + G)]
            if mem.max() < 0:
                continue
            nk = min(keep, min(int(mem.max()) // Bs + 1, NB))
            n += int(np.clip(np.minimum(nk * Bs, np.minimum(mem + 1, L)), 0, None).sum())
    return n


def block_pairs(prob, Bs, keep):
    """(coarse pairs: queries x eligible pooled blocks, refine pairs: queries x kept tokens)."""
    import numpy as np
    coarse = refine = 0
    for b in range(prob.B):
        pos = prob.q_pos[b].astype(np.int64)
        NB = -(-int(prob.k_len[b]) // Bs)
        elig = np.where(pos < 0, 0, np.minimum(pos // Bs + 1, NB))
        coarse += int(elig.sum())
        refine += int(np.minimum(elig, keep).sum() * Bs)
    return coarse, refine


def filtered_decode_bytes(prob, spec):
    """Algorithmic HBM bytes of one block-filtered decode step: (coarse: each sequence's pooled
    block keys read once, bf16 or fp32 for fp32 caches; refine: each token list's keys, + its
    fp32 scale for FP8 caches, read once: a list per query for the block path, per group for the
    group path, of min(keep, eligible blocks) blocks cut to the cache)."""
    import numpy as np
    import workloads as W
    Bs, keep = spec["block_size"], spec["n_blocks_keep"]
    G = spec.get("group_size", 1) if spec["op"] == "gblock" else 1
    kb = {W.F32: 4, W.BF16: 2, W.FP8_E4M3: 1}[prob.k_dtype]
    tok = prob.D * kb + (4 if prob.k_dtype == W.FP8_E4M3 else 0)
    pooled_b = prob.D * (4 if prob.k_dtype == W.F32 else 2)
    coarse = refine = 0
    for b in range(prob.B):
        pos = prob.q_pos[b].astype(np.int64)
        L = int(prob.k_len[b])
        NB = -(-L // Bs)
        if pos.max() >= 0:
            coarse += min(NB, int(pos.max()) // Bs + 1) * pooled_b
        for g in range((prob.T + G - 1) // G):
            top = int(pos[g * G:min(prob.T, g * G + G)].max())
            if top >= 0:
                nk = min(keep, min(top // Bs + 1, NB))
                refine += min(nk * Bs, L) * tok
    return coarse, refine


# ----------------------------------------------------------------------------------------------

def cpu_oracle_baseline(name, spec, prob, budget_s=12.0):
    """Times the oracle on a bounded, evenly spaced row sample of the workload."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    op = spec["op"]
    inp = oracle.Inputs(prob) if op != "latent" else None    # latent rows convert per sequence
    B, T = prob.B, prob.T
    done_pairs = 0
    rows = 0
    t0 = time.perf_counter()
    if op == "dense":
        stride = max(1, T // 64)
        order = [(b, t) for off in range(stride) for t in range(T - 1 - off, -1, -stride)
                 for b in range(B)]
        for b, t in order:
            oracle.dense_row(inp, b, t, spec["k"])
            done_pairs += inp.P(b, t)
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = (f"{rows} query rows of {B * T} (interleaved with stride {stride} from the last "
                  "row), full prefix each")
    elif op == "group":
        G, C = spec["group_size"], spec["n_cand"]
        NG = (T + G - 1) // G
        stride = max(1, NG // 64)
        for b, g in [(b, g) for off in range(stride) for g in range(NG - 1 - off, -1, -stride) for b in range(B)]:
            ps = oracle.group_proxy_scan(inp, b, g, G, C)
            for t in oracle.group_members(T, G, g):
                oracle.refine_row(inp, b, t, spec["k"], ps["cand"])
                done_pairs += inp.P(b, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {B * T} in whole groups, interleaved with stride {stride} (proxy scan + refine)"
    elif op == "reuse":
        G = spec["group_size"]
        NG = (T + G - 1) // G
        stride = max(1, NG // 64)
        for b, g in [(b, g) for off in range(stride) for g in range(NG - 1 - off, -1, -stride) for b in range(B)]:
            ps = oracle.group_proxy_scan(inp, b, g, G, spec["k"])
            for t in oracle.group_members(T, G, g):
                oracle.reuse_row(inp, b, t, ps)
                done_pairs += inp.P(b, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {B * T} in whole groups, interleaved with stride {stride} (proxy scan + reuse)"
    elif op == "gblock":
        G, Bs, keep = spec["group_size"], spec["block_size"], spec["n_blocks_keep"]
        NG = (T + G - 1) // G
        pooled = {}
        stride = max(1, NG // 64)
        for b, g in [(b, g) for off in range(stride) for g in range(NG - 1 - off, -1, -stride)
                     for b in range(B)]:
            if b not in pooled:
                pooled[b] = oracle.pool_keys(prob, b, Bs)
            gs = oracle.group_block_scan(inp, b, g, G, Bs, keep, pooled[b])
            for t in oracle.group_members(T, G, g):
                oracle.refine_row(inp, b, t, spec["k"], gs["tokens"])
                done_pairs += inp.P(b, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = (f"{rows} query rows of {B * T} in whole groups, interleaved with stride {stride} "
                  f"(pooling each of {len(pooled)} sequences once, proxy block scan + refine)")
    elif op == "latent":
        # the absorbed queries of the sampled rows, then the dense oracle on them
        stride = max(1, T // 64)
        order = [(b, t) for b in range(B) for off in range(stride) for t in range(T - 1 - off, -1, -stride)]
        cur_b, lat = -1, None
        for b, t in order:
            if b != cur_b:                     # the sequence's latent rows in float64
                ks = None if prob.k_scale is None else prob.k_scale[b]
                cur_b, lat = b, oracle.keys_f64(prob.k[b], prob.k_dtype, ks)
            a = oracle.absorb_queries(prob.q[b, t], prob.q_dtype, prob.wk)
            P = oracle.visible_len(int(prob.q_pos[b, t]), int(prob.k_len[b]))
            sc = oracle.index_scores(oracle.bf16_bits_to_f64(a["bits"]), prob.w[b, t].astype(np.float64), lat[:P])
            oracle.select_topk(sc, np.arange(P, dtype=np.int64), spec["k"])
            done_pairs += P
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = (f"{rows} query rows of {B * T} (sequence by sequence, stride {stride} from the last "
                  "row): absorbed queries + full latent prefix each")
    elif op == "given":
        G = spec["group_size"]
        banks = W.make_banks(prob, G, spec["n_cand"], 0)
        stride = max(1, T // 128)
        for t in [t for off in range(stride) for t in range(T - 1 - off, -1, -stride)]:
            v = banks[0, t // G]
            oracle.refine_row(inp, 0, t, spec["k"], np.unique(v[v >= 0]))
            done_pairs += inp.P(0, t)
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {T} (interleaved with stride {stride}), refine over the given bank"
    else:
        Bs, keep = spec["block_size"], spec["n_blocks_keep"]
        pooled = {}
        stride = max(1, T // 128)
        for b, t in [(b, t) for off in range(stride) for t in range(T - 1 - off, -1, -stride)
                     for b in range(B)]:
            if b not in pooled:
                pooled[b] = oracle.pool_keys(prob, b, Bs)
            oracle.block_row(inp, b, t, spec["k"], Bs, keep, pooled[b])
            done_pairs += inp.P(b, t)
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = (f"{rows} query rows of {B * T} (interleaved with stride {stride}), pooling each of "
                  f"{len(pooled)} sequences once + coarse + refine")
    dt = time.perf_counter() - t0
    return {"value": done_pairs / dt, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": sample + f"; {dt:.1f} s; dense-equivalent pairs", **host_info(threads)}


def host_info(blas_threads):
    """The host the oracle ran on: logical CPUs of the machine and of this process, the BLAS
    thread count the oracle's matrix products used (= `cores`), and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return {"host_nproc": os.cpu_count() or 1, "host_cpus_available": avail,
            "oracle_threads": int(blas_threads), "cpu_model": model}




# ----------------------------------------------------------------------------------------------

class Run:
    """One workload on the GPU: inputs in HBM, outputs and workspace allocated once, `step()`
    enqueues one full indexer call."""

    def __init__(self, name, seed):
        import torch
        import workloads as W
        import sparse_attention_indexer_02_amd as idx
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from gpu_util import dev
        self.name, self.seed = name, seed
        self.spec = spec = W.WORKLOADS[name]
        log(f"[bench] generating {name} (seed {seed})")
        self.prob = prob = spec["gen"](seed)
        self.t = t = dev(prob, "cuda:0")
        self.k = k = spec["k"]
        B, T = prob.B, prob.T
        self.op = op = spec["op"]
        self.out_idx = torch.empty((B, T, k), dtype=torch.int32, device="cuda:0")
        self.out_sc = torch.empty((B, T, k), dtype=torch.float32, device="cuda:0")
        self.q_lat = None
        if op == "latent":
            self.q_lat = torch.empty((B, T, prob.H, prob.k.shape[2]), dtype=torch.bfloat16, device="cuda:0")
        p = idx.make_problem(t["q"] if self.q_lat is None else self.q_lat, t["k"], t["w"], t["q_pos"],
                             t["k_len"], t["k_scale"], t["q_scale"])
        self.banks_np = None
        if op in ("dense", "latent"):
            need = idx.workspace_bytes(idx.OP_SCORE_TOPK, p, k)
        elif op == "group":
            need = idx.workspace_bytes(idx.OP_GROUP, p, k, spec["group_size"], spec["n_cand"])
        elif op == "reuse":
            need = idx.workspace_bytes(idx.OP_REUSE, p, k, spec["group_size"], 0)
        elif op == "gblock":
            need = int(idx.lib().idx_group_block_workspace_bytes(ctypes.byref(p), k, spec["group_size"],
                                                                  spec["block_size"], spec["n_blocks_keep"]))
        elif op == "given":
            self.banks_np = W.make_banks(prob, spec["group_size"], spec["n_cand"], seed)
            self.banks = torch.from_numpy(self.banks_np).to("cuda:0")
            need = idx.workspace_bytes(idx.OP_REFINE, p, k, spec["group_size"], spec["n_cand"])
        else:
            need = idx.workspace_bytes(idx.OP_BLOCK, p, k, spec["block_size"], spec["n_blocks_keep"])
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        # pooled block keys kept beside the cache (a decoding server pools a block once, when it
        # is complete): pooled here once, before timing; the pooling of the whole cache is timed
        # on its own
        self.pooled = None
        if spec.get("pooled"):
            self.pooled = idx.block_pool(t["k"], spec["block_size"], k_len=t["k_len"], k_scale=t["k_scale"])

    def step(self):
        import sparse_attention_indexer_02_amd as idx
        t, k, spec, op = self.t, self.k, self.spec, self.op
        kw = dict(k_len=t["k_len"], out_idx=self.out_idx, out_score=self.out_sc, workspace=self.ws)
        if op == "dense":
            idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_scale=t["k_scale"],
                           q_scale=t["q_scale"], **kw)
        elif op == "latent":
            idx.absorb_queries(t["q"], t["wk"], out=self.q_lat)
            idx.score_topk(self.q_lat, t["k"], t["w"], t["q_pos"], topk=k, k_scale=t["k_scale"], **kw)
        elif op == "group":
            idx.group_proxy_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                   group_size=spec["group_size"], n_cand=spec["n_cand"],
                                   k_scale=t["k_scale"], **kw)
        elif op == "gblock":
            idx.group_block_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                   group_size=spec["group_size"], block_size=spec["block_size"],
                                   n_blocks_keep=spec["n_blocks_keep"], k_scale=t["k_scale"],
                                   pooled=self.pooled, **kw)
        elif op == "reuse":
            idx.group_proxy_reuse(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                  group_size=spec["group_size"], k_scale=t["k_scale"], **kw)
        elif op == "given":
            idx.refine_given(t["q"], t["k"], t["w"], t["q_pos"], self.banks, topk=k,
                             group_size=spec["group_size"], k_scale=t["k_scale"], **kw)
        else:
            idx.block_coarse_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                    block_size=spec["block_size"],
                                    n_blocks_keep=spec["n_blocks_keep"], k_scale=t["k_scale"],
                                    pooled=self.pooled, **kw)

    def time(self, steps, warmup):
        """Mean step time: HIP events around exactly `steps` steps after `warmup` untimed ones,
        with the library's per-kernel timers off (their events between launches add several
        microseconds per kernel to a short step). The per-kernel durations (the roofline's mean
        launch time) come from a second pass of `steps` steps with the timers on."""
        import torch
        import sparse_attention_indexer_02_amd as idx
        log(f"[bench] {self.name}: warmup {warmup}")
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        log(f"[bench] {self.name}: timing {steps} steps")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - w0
        self.ms_step = e0.elapsed_time(e1) / steps
        self.steps = steps
        # kernel pass: the same steps with an event pair around every launch
        idx.timer_enable(True)
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        self.ms_step_events = e0.elapsed_time(e1) / steps
        self.kernels = {n: idx.timer_read(n)
                        for n in ("score", "topk", "sort", "proxy", "pool", "block_refine", "reuse",
                                  "decode_scan", "decode_select", "absorb")}
        idx.timer_enable(False)
        log(f"[bench] {self.name}: {self.ms_step:.4f} ms/step ({self.ms_step_events:.4f} with kernel events); "
            "per-kernel ms/step: " + ", ".join(
                f"{n} {ms / steps:.3f} ({c // max(1, steps)} launches)"
                for n, (ms, c) in self.kernels.items() if c))
        self.pool_ms = None
        if self.pooled is not None:
            t, spec = self.t, self.spec
            e0.record()
            for _ in range(steps):
                idx.block_pool(t["k"], spec["block_size"], k_len=t["k_len"], k_scale=t["k_scale"],
                               out=self.pooled)
            e1.record()
            torch.cuda.synchronize()
            self.pool_ms = e0.elapsed_time(e1) / steps
            log(f"[bench] {self.name}: pooling the whole cache (outside the step) {self.pool_ms:.4f} ms")

    def _mfma(self, kernel, flops, **extra):
        import workloads as W
        ms, n = self.kernels["block_refine" if kernel.startswith("block_refine") else "score"]
        per_launch = flops / (n / self.steps)
        achieved = per_launch / (ms / n * 1e-3) / 1e12
        # FP8 queries (with FP8 keys) run on the FP8 matrix cores: their own peak
        peak = PEAK_FP8_TFLOPS if self.prob.q_dtype == W.FP8_E4M3 else PEAK_BF16_TFLOPS
        return {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": measured_traffic(self.name, kernel),
                "per_launch": f"{per_launch:.4g} flop", "mean_launch_ms": ms / n, **extra}

    def report(self):
        """(config, roofline) of the timed run."""
        import workloads as W
        prob, spec, op = self.prob, self.spec, self.op
        cfg = {"workload": self.name, "B": prob.B, "T": prob.T, "H": prob.H, "D": prob.D,
               "N": prob.N, "k": self.k, "q_dtype": W.DTYPE_NAMES[prob.q_dtype],
               "k_dtype": W.DTYPE_NAMES[prob.k_dtype], "seed": self.seed,
               "pairs_per_step": prob.pairs()}
        if op == "latent":
            cfg.update(latent_width=prob.k.shape[2],
                       absorb_ms_per_step=self.kernels["absorb"][0] / self.steps)
        if op in ("dense", "latent") and self.kernels["decode_scan"][1] == 0:
            roof = self._mfma("score_kernel", dense_flops(prob))
        elif op in ("dense", "latent"):
            # decode shape: the streaming scan is the dominant kernel, bound by the key-cache read
            ms, n = self.kernels["decode_scan"]
            byts = decode_bytes(prob)
            per_launch = byts / (n / self.steps)
            achieved = per_launch / (ms / n * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": "decode_scan_kernel", "achieved": achieved,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                    "traffic": measured_traffic(self.name, "decode_scan_kernel"),
                    "per_launch": f"{per_launch:.4g} B", "mean_launch_ms": ms / n}
        elif op in ("group", "reuse") and self.kernels["decode_scan"][1]:
            # decode-shaped groups: the proxies' scan is the decode scan, bound by the cache read
            ms, n = self.kernels["decode_scan"]
            byts = decode_bytes(prob)
            per_launch = byts / (n / self.steps)
            achieved = per_launch / (ms / n * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": "decode_scan_kernel", "achieved": achieved,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                    "traffic": measured_traffic(self.name, "decode_scan_kernel"),
                    "per_launch": f"{per_launch:.4g} B (the proxies' scan of the cache)",
                    "mean_launch_ms": ms / n}
            cfg.update(group_size=spec["group_size"])
            if op == "group":
                cfg.update(n_cand=spec["n_cand"])
        elif op == "group":
            pp, rp = group_refine_pairs(prob, spec["group_size"], spec["n_cand"])
            roof = self._mfma("score_kernel", 2.0 * prob.H * prob.D * (pp + rp))
            cfg.update(group_size=spec["group_size"], n_cand=spec["n_cand"],
                       algorithmic_pairs_per_step=pp + rp)
        elif spec.get("pooled"):
            # block filter at decode: the decode scan streams the kept tokens once per list, bound
            # by their read; the coarse scan of the pooled keys is reported beside it
            cb, rb = filtered_decode_bytes(prob, spec)
            ms, n = self.kernels["decode_scan"]
            if n:
                kern, per_launch = "decode_scan_kernel", rb / (n / self.steps)
                achieved = per_launch / (ms / n * 1e-3) / 1e9
                extra = {"per_launch": f"{per_launch:.4g} B (kept tokens' keys and scales)"}
            else:
                ms, n = self.kernels["score"]
                kern = "score_kernel"
                achieved = (cb + rb) / (ms / self.steps * 1e-3) / 1e9
                extra = {"per_step": f"{cb + rb:.4g} B over {n // self.steps} launches (pooled keys and "
                                     "kept tokens)"}
            cms, cn = self.kernels["score"]
            roof = {"bound": "hbm", "kernel": kern, "achieved": achieved,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                    "traffic": measured_traffic(self.name, kern), "mean_launch_ms": ms / n, **extra,
                    "coarse_scan": {"bytes_per_step": cb, "ms_per_step": cms / self.steps,
                                    "launches_per_step": cn // self.steps}}
            G = spec.get("group_size", 1) if op == "gblock" else 1
            cfg.update(block_size=spec["block_size"], n_blocks_keep=spec["n_blocks_keep"],
                       pooled_keys="kept beside the cache, not pooled in the step",
                       pool_whole_cache_ms=self.pool_ms)
            if op == "gblock":
                cfg.update(group_size=G)
        elif op == "gblock":
            G, Bs, keep = spec["group_size"], spec["block_size"], spec["n_blocks_keep"]
            rp = gblock_refine_pairs(prob, G, Bs, keep)
            roof = self._mfma("score_kernel", 2.0 * prob.H * prob.D * rp,
                              note="score kernel time covers the proxies' block scan and the member "
                                   "refine; the flops are the refine's")
            cfg.update(group_size=G, block_size=Bs, n_blocks_keep=keep, algorithmic_pairs_per_step=rp)
        elif op == "reuse":
            pp, _ = group_refine_pairs(prob, spec["group_size"], 1)
            roof = self._mfma("score_kernel", 2.0 * prob.H * prob.D * pp)
            cfg.update(group_size=spec["group_size"], algorithmic_pairs_per_step=pp)
        elif op == "given":
            rp = given_pairs(prob, spec["group_size"], self.banks_np)
            roof = self._mfma("score_kernel", 2.0 * prob.H * prob.D * rp)
            cfg.update(group_size=spec["group_size"], n_cand=spec["n_cand"], algorithmic_pairs_per_step=rp)
        else:
            cp, rp = block_pairs(prob, spec["block_size"], spec["n_blocks_keep"])
            roof = self._mfma(block_refine_kernel_name(prob, spec["block_size"]),
                              2.0 * prob.H * prob.D * rp)
            cfg.update(block_size=spec["block_size"], n_blocks_keep=spec["n_blocks_keep"],
                       algorithmic_pairs_per_step=cp + rp)
        cfg["kernel_ms_per_step"] = {n_: round(ms_ / self.steps, 4)
                                     for n_, (ms_, c) in self.kernels.items() if c}
        cfg["kernel_pass_ms_per_step"] = round(self.ms_step_events, 4)
        return cfg, roof

    def recall_vs_dense(self):
        """recall@k of the last step's selections against the dense indexer's GPU selection on
        the same inputs: |S_variant & S_dense| / |S_dense| summed over every query row. The dense
        path is the one the parity tests check against the oracle."""
        import torch
        import sparse_attention_indexer_02_amd as idx
        t = self.t
        d_idx, _ = idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=self.k, k_len=t["k_len"],
                                  k_scale=t["k_scale"], want_score=False)
        v = self.out_idx.reshape(-1, self.k)
        d = d_idx.reshape(-1, self.k)
        hit = tot = 0
        for r0 in range(0, v.shape[0], 2048):
            vs = torch.sort(v[r0:r0 + 2048], dim=-1).values.contiguous()
            ds = torch.sort(d[r0:r0 + 2048], dim=-1).values.contiguous()
            pos = torch.searchsorted(vs, ds).clamp_(max=self.k - 1)
            found = (torch.gather(vs, 1, pos) == ds) & (ds >= 0)
            hit += int(found.sum())
            tot += int((ds >= 0).sum())
        torch.cuda.synchronize()
        return {"recall_at_k": hit / max(1, tot), "rows": int(v.shape[0]), "dense_selected": tot,
                "reference": "dense indexer (idx_score_topk) on the same inputs, GPU"}

    def line(self, cpu=True, recall=True):
        """The workload's numbers: ms/step, pairs/s, rows/s, roofline, oracle baseline."""
        cfg, roof = self.report()
        prob = self.prob
        out = {"ms_per_step": self.ms_step, "value": prob.pairs() / (self.ms_step * 1e-3),
               "unit": "pairs/s", "topk_rows_per_s": prob.B * prob.T / (self.ms_step * 1e-3),
               "config": cfg, "roofline": roof, "wall_s_timed": self.wall}
        if recall and self.op not in ("dense", "latent"):
            log(f"[bench] {self.name}: recall vs the dense indexer")
            out["recall_vs_dense"] = self.recall_vs_dense()
        out["cpu_baseline"] = None
        if cpu:
            log(f"[bench] {self.name}: timing the CPU oracle on a row sample")
            out["cpu_baseline"] = cpu_oracle_baseline(self.name, self.spec, prob)
        return out

    def free(self):
        import torch
        for a in ("t", "out_idx", "out_sc", "ws", "banks", "pooled", "q_lat"):
            if hasattr(self, a):
                delattr(self, a)
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="one workload alone (default: the headline, dense64k with decode128k)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-recall", action="store_true",
                    help="skip the recall check against the dense indexer (it launches the dense path "
                         "after the timed steps; profiles of the timed kernels leave it out)")
    ap.add_argument("--copy-probe", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the indexer here is "
              "single-GPU by design", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    headline = args.workload is None
    name = "dense64k" if headline else args.workload
    run = Run(name, args.seed)
    run.time(args.steps, args.warmup)
    main_line = run.line(cpu=not args.no_cpu, recall=not args.no_recall)
    q_dtype = run.prob.q_dtype
    run.free()
    import workloads as W
    out = {"metric": METRIC, "value": main_line["value"], "unit": "pairs/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_line["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {W.BF16: "bf16", W.FP8_E4M3: "fp8 (e4m3 queries and keys, fp32 accumulate)"}.get(q_dtype, "f32"),
           "data": "synthetic (seeded generators shaped like the pages' workloads)"}
    out.update({k_: v_ for k_, v_ in main_line.items() if k_ not in out})
    if headline:
        dec = Run("decode128k", args.seed)
        dec.time(args.steps, args.warmup)
        d = dec.line(cpu=not args.no_cpu, recall=not args.no_recall)
        d["dtype"] = "bf16 queries x fp8 e4m3 keys (bf16 MFMA, fp32 accumulate)"
        d["steps"], d["warmup"] = args.steps, args.warmup
        out["decode128k"] = d
        dec.free()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
