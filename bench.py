"""Benchmark of the MI355X DSA lightning indexer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense16k] [--no-cpu]
    python bench.py --copy-probe BYTES     (a plain device copy of known size, for calibrating
                                            the HBM byte counters of rocprofv3 --pmc)

One step = one full indexer call (every stage of the path: scoring, masking, top-k selection,
and for the variants the proxy / pooling / candidate stages) over one batch of seeded synthetic
input that is already resident in HBM. Prints ONE JSON line.

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
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# source files each profiled kernel is compiled from (its own file and the headers it includes)
KERNEL_SOURCES = {
    "score_kernel": ["score.hip", "score_tile.h", "common.h", "kernels.h"],
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
    return 2.0 * prob.H * prob.D * prob.pairs()


def decode_bytes(prob):
    import numpy as np
    kl = prob.k_len.astype(np.int64)
    kb = prob.D * (1 if prob.k_dtype == 2 else (2 if prob.k_dtype == 1 else 4))
    per_tok = kb + (4 if prob.k_dtype == 2 else 0)
    return float((kl * per_tok).sum() + prob.q.nbytes + prob.w.nbytes)


def group_refine_pairs(prob, G, C):
    """Pairs scored by the group path: proxy full-prefix scans + member refines over C."""
    import numpy as np
    T = prob.T
    NG = (T + G - 1) // G
    pos = prob.q_pos[0].astype(np.int64)
    L = int(prob.k_len[0])
    proxy = sum(min(int(pos[min(T, (g + 1) * G) - 1]) + 1, L) for g in range(NG))
    refine = sum(min(C, min(int(pos[min(T, (g + 1) * G) - 1]) + 1, L)) * (min(T, (g + 1) * G) - g * G)
                 for g in range(NG))
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
    pos = prob.q_pos[0].astype(np.int64)
    L = int(prob.k_len[0])
    NB = -(-L // Bs)
    n = 0
    for g in range((prob.T + G - 1) // G):
        mem = pos[g * G:min(prob.T, g * G + G)]
        nk = min(keep, min(int(mem.max()) // Bs + 1, NB))
        n += int(np.minimum(nk * Bs, np.minimum(mem + 1, L)).sum())
    return n


def block_pairs(prob, Bs, keep):
    import numpy as np
    pos = prob.q_pos[0].astype(np.int64)
    NB = -(-int(prob.k_len[0]) // Bs)
    coarse = int(np.minimum(pos // Bs + 1, NB).sum())
    refine = int(np.minimum(np.minimum(pos // Bs + 1, NB), keep).sum() * Bs)
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
    inp = oracle.Inputs(prob)
    B, T = prob.B, prob.T
    op = spec["op"]
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
        for g in [g for off in range(stride) for g in range(NG - 1 - off, -1, -stride)]:
            ps = oracle.group_proxy_scan(inp, 0, g, G, C)
            for t in oracle.group_members(T, G, g):
                oracle.refine_row(inp, 0, t, spec["k"], ps["cand"])
                done_pairs += inp.P(0, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {T} in whole groups, interleaved with stride {stride} (proxy scan + refine)"
    elif op == "reuse":
        G = spec["group_size"]
        NG = (T + G - 1) // G
        stride = max(1, NG // 64)
        for g in [g for off in range(stride) for g in range(NG - 1 - off, -1, -stride)]:
            ps = oracle.group_proxy_scan(inp, 0, g, G, spec["k"])
            for t in oracle.group_members(T, G, g):
                oracle.reuse_row(inp, 0, t, ps)
                done_pairs += inp.P(0, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {T} in whole groups, interleaved with stride {stride} (proxy scan + reuse)"
    elif op == "gblock":
        G, Bs, keep = spec["group_size"], spec["block_size"], spec["n_blocks_keep"]
        NG = (T + G - 1) // G
        pooled = oracle.pool_keys(prob, 0, Bs)
        stride = max(1, NG // 64)
        for g in [g for off in range(stride) for g in range(NG - 1 - off, -1, -stride)]:
            gs = oracle.group_block_scan(inp, 0, g, G, Bs, keep, pooled)
            for t in oracle.group_members(T, G, g):
                oracle.refine_row(inp, 0, t, spec["k"], gs["tokens"])
                done_pairs += inp.P(0, t)
                rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = (f"{rows} query rows of {T} in whole groups, interleaved with stride {stride} "
                  "(pooling once, proxy block scan + refine)")
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
        pooled = oracle.pool_keys(prob, 0, Bs)
        stride = max(1, T // 128)
        for t in [t for off in range(stride) for t in range(T - 1 - off, -1, -stride)]:
            oracle.block_row(inp, 0, t, spec["k"], Bs, keep, pooled)
            done_pairs += inp.P(0, t)
            rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
        sample = f"{rows} query rows of {T} (interleaved with stride {stride}), pooling + coarse + refine"
    dt = time.perf_counter() - t0
    return {"value": done_pairs / dt, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": sample + f"; {dt:.1f} s; dense-equivalent pairs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense16k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the indexer here is "
              "single-GPU by design", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import numpy as np
    import torch
    import workloads as W
    import sparse_attention_indexer_02_amd as idx
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import dev

    spec = W.WORKLOADS[args.workload]
    log(f"[bench] generating {args.workload} (seed {args.seed})")
    prob = spec["gen"](args.seed)
    t = dev(prob, "cuda:0")
    k = spec["k"]
    B, T = prob.B, prob.T
    op = spec["op"]
    out_idx = torch.empty((B, T, k), dtype=torch.int32, device="cuda:0")
    out_sc = torch.empty((B, T, k), dtype=torch.float32, device="cuda:0")
    p = idx.make_problem(t["q"], t["k"], t["w"], t["q_pos"], t["k_len"], t["k_scale"])
    if op == "dense":
        need = idx.workspace_bytes(idx.OP_SCORE_TOPK, p, k)
    elif op == "group":
        need = idx.workspace_bytes(idx.OP_GROUP, p, k, spec["group_size"], spec["n_cand"])
    elif op == "reuse":
        need = idx.workspace_bytes(idx.OP_REUSE, p, k, spec["group_size"], 0)
    elif op == "gblock":
        need = int(idx.lib().idx_group_block_workspace_bytes(ctypes.byref(p), k, spec["group_size"],
                                                              spec["block_size"], spec["n_blocks_keep"]))
    elif op == "given":
        banks_np = W.make_banks(prob, spec["group_size"], spec["n_cand"], args.seed)
        banks = torch.from_numpy(banks_np).to("cuda:0")
        need = idx.workspace_bytes(idx.OP_REFINE, p, k, spec["group_size"], spec["n_cand"])
    else:
        need = idx.workspace_bytes(idx.OP_BLOCK, p, k, spec["block_size"], spec["n_blocks_keep"])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        if op == "dense":
            idx.score_topk(t["q"], t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"],
                           k_scale=t["k_scale"], out_idx=out_idx, out_score=out_sc, workspace=ws)
        elif op == "group":
            idx.group_proxy_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                   group_size=spec["group_size"], n_cand=spec["n_cand"],
                                   k_len=t["k_len"], k_scale=t["k_scale"], out_idx=out_idx,
                                   out_score=out_sc, workspace=ws)
        elif op == "gblock":
            idx.group_block_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                   group_size=spec["group_size"], block_size=spec["block_size"],
                                   n_blocks_keep=spec["n_blocks_keep"], k_len=t["k_len"],
                                   out_idx=out_idx, out_score=out_sc, workspace=ws)
        elif op == "reuse":
            idx.group_proxy_reuse(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                  group_size=spec["group_size"], k_len=t["k_len"],
                                  k_scale=t["k_scale"], out_idx=out_idx, out_score=out_sc,
                                  workspace=ws)
        elif op == "given":
            idx.refine_given(t["q"], t["k"], t["w"], t["q_pos"], banks, topk=k,
                             group_size=spec["group_size"], k_len=t["k_len"], k_scale=t["k_scale"],
                             out_idx=out_idx, out_score=out_sc, workspace=ws)
        else:
            idx.block_coarse_refine(t["q"], t["k"], t["w"], t["q_pos"], topk=k,
                                    block_size=spec["block_size"],
                                    n_blocks_keep=spec["n_blocks_keep"], k_len=t["k_len"],
                                    out_idx=out_idx, out_score=out_sc, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    idx.timer_enable(True)
    log(f"[bench] timing {args.steps} steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    kernels = {name: idx.timer_read(name)
               for name in ("score", "topk", "sort", "proxy", "pool", "block_refine", "reuse",
                            "decode_scan", "decode_select")}
    idx.timer_enable(False)
    log("[bench] per-kernel ms/step: " + ", ".join(
        f"{n} {ms / args.steps:.3f} ({c // max(1, args.steps)} launches)" for n, (ms, c) in kernels.items() if c))

    pairs = prob.pairs()
    value = pairs / (ms_step * 1e-3)
    rows_per_s = B * T / (ms_step * 1e-3)
    cfg = {"workload": args.workload, "B": B, "T": T, "H": prob.H, "D": prob.D, "N": prob.N,
           "k": k, "q_dtype": W.DTYPE_NAMES[prob.q_dtype], "k_dtype": W.DTYPE_NAMES[prob.k_dtype],
           "seed": args.seed, "pairs_per_step": pairs}
    if op == "dense" and kernels["decode_scan"][1] == 0:
        dom = "score"
        ms, n = kernels["score"]
        flops = dense_flops(prob)
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "score_kernel", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, "score_kernel"),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n}
    elif op == "dense":
        # decode shape: the streaming scan is the dominant kernel, bound by the key-cache read
        ms, n = kernels["decode_scan"]
        byts = decode_bytes(prob)
        achieved = byts / (n / args.steps) / (ms / n * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "decode_scan_kernel", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(args.workload, "decode_scan_kernel"),
                "per_launch": f"{byts / (n / args.steps):.4g} B",
                "mean_launch_ms": ms / n}
    elif op == "group":
        pp, rp = group_refine_pairs(prob, spec["group_size"], spec["n_cand"])
        ms, n = kernels["score"]
        flops = 2.0 * prob.H * prob.D * (pp + rp)
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "score_kernel", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, "score_kernel"),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n}
        cfg.update(group_size=spec["group_size"], n_cand=spec["n_cand"],
                   algorithmic_pairs_per_step=pp + rp)
    elif op == "gblock":
        G, Bs, keep = spec["group_size"], spec["block_size"], spec["n_blocks_keep"]
        rp = gblock_refine_pairs(prob, G, Bs, keep)
        ms, n = kernels["score"]
        flops = 2.0 * prob.H * prob.D * rp
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "score_kernel", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, "score_kernel"),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n,
                "note": "score kernel time covers the proxies' block scan and the member refine; "
                        "the flops are the refine's"}
        cfg.update(group_size=G, block_size=Bs, n_blocks_keep=keep, algorithmic_pairs_per_step=rp)
    elif op == "reuse":
        pp, _ = group_refine_pairs(prob, spec["group_size"], 1)
        ms, n = kernels["score"]
        flops = 2.0 * prob.H * prob.D * pp
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "score_kernel", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, "score_kernel"),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n}
        cfg.update(group_size=spec["group_size"], algorithmic_pairs_per_step=pp)
    elif op == "given":
        rp = given_pairs(prob, spec["group_size"], banks_np)
        ms, n = kernels["score"]
        flops = 2.0 * prob.H * prob.D * rp
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "score_kernel", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, "score_kernel"),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n}
        cfg.update(group_size=spec["group_size"], n_cand=spec["n_cand"], algorithmic_pairs_per_step=rp)
    else:
        cp, rp = block_pairs(prob, spec["block_size"], spec["n_blocks_keep"])
        ms, n = kernels["block_refine"]
        flops = 2.0 * prob.H * prob.D * rp
        achieved = flops / (n / args.steps) / (ms / n * 1e-3) / 1e12
        kname = block_refine_kernel_name(prob, spec["block_size"])
        roof = {"bound": "mfma", "kernel": kname, "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(args.workload, kname),
                "per_launch": f"{flops / (n / args.steps):.4g} flop", "mean_launch_ms": ms / n}
        cfg.update(block_size=spec["block_size"], n_blocks_keep=spec["n_blocks_keep"],
                   algorithmic_pairs_per_step=cp + rp)
    cfg["kernel_ms_per_step"] = {n_: round(ms_ / args.steps, 4) for n_, (ms_, c) in kernels.items() if c}

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a row sample")
        cpu = cpu_oracle_baseline(args.workload, spec, prob)

    out = {"metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if prob.q_dtype == W.BF16 else "f32",
           "data": "synthetic (seeded generators shaped like the pages' workloads)",
           "config": cfg, "topk_rows_per_s": rows_per_s, "roofline": roof, "cpu_baseline": cpu,
           "wall_s_timed": wall}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
