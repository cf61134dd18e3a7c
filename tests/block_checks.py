"""Checks shared by the block-path GPU tests: the GPU's kept blocks against the oracle's
pooled-block scores (tie band at the n_keep-th score), and each final row against the oracle's
token scores over the tokens of the GPU's own kept blocks (test helper)."""
import numpy as np

import oracle
from gpu_util import say
from parity import check_selection


def check_block(prob, k, Bs, keep, gi, gs, gb, rows, name):
    inp = oracle.Inputs(prob)
    pooled = {}
    e2e_diff = e2e_tot = 0
    for b, t in rows:
        if b not in pooled:
            pooled[b] = oracle.pool_keys(prob, b, Bs)
        r = oracle.block_row(inp, b, t, k, Bs, keep, pooled[b])
        n_elig = len(r["block_scores"])
        check_selection(gb[b, t], None, np.arange(n_elig), r["block_scores"],
                        r["block_magnitude"], keep, prob.D, ctx=f"{name} blocks b{b} t{t}",
                        oracle_sel=r["blocks"])
        kept = gb[b, t, :min(keep, n_elig)].astype(np.int64)
        assert (np.diff(kept) > 0).all() and (gb[b, t, min(keep, n_elig):] == -1).all()
        d = oracle.dense_row(inp, b, t, k)
        toks = np.sort((kept[:, None] * Bs + np.arange(Bs)[None]).reshape(-1))
        toks = toks[toks < inp.P(b, t)]
        check_selection(gi[b, t], gs[b, t], toks, d["all_scores"][toks], d["magnitude"][toks],
                        k, prob.D, ctx=f"{name} b{b} t{t}")
        sel = gi[b, t][gi[b, t] >= 0]
        e2e_diff += len(np.setxor1d(sel, r["ids"])) // 2
        e2e_tot += len(r["ids"])
    say(f"{name}: end-to-end differences vs oracle {e2e_diff}/{e2e_tot}")


def check_gb(prob, k, G, Bs, keep, gi, gs, gb, groups, name):
    inp = oracle.Inputs(prob)
    pooled = {b: oracle.pool_keys(prob, b, Bs) for b in {b for b, _ in groups}}
    for b, g in groups:
        sc = oracle.group_block_scan(inp, b, g, G, Bs, keep, pooled[b])
        n_elig = len(sc["block_scores"])
        check_selection(gb[b, g], None, np.arange(n_elig), sc["block_scores"], sc["block_magnitude"],
                        keep, prob.D, ctx=f"{name} blocks b{b} g{g}", oracle_sel=sc["blocks"])
        kept = gb[b, g][gb[b, g] >= 0].astype(np.int64)
        assert (np.diff(kept) > 0).all()
        toks = (kept[:, None] * Bs + np.arange(Bs)[None]).reshape(-1)
        for t in oracle.group_members(prob.T, G, g):
            # the oracle's token scores over the GPU's own kept blocks (inside the prefix)
            r = oracle.refine_row(inp, b, t, k, toks)
            check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"], k,
                            prob.D, ctx=f"{name} b{b} t{t}")
