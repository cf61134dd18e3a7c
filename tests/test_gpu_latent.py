"""GPU parity of absorbed-query scoring of a shared latent cache ("LatentIndex: Cross-Layer Sharing
with Layer-Specific Selection for Sparse Attention", abstract). Stage-wise, as for the other
multi-stage paths: the absorbed queries against the oracle's exact values (each element a valid
bf16 rounding of a value within the fp32 accumulation bound, nearly all equal to the oracle's
own rounding), then the selection against the oracle's dense indexer on the GPU's absorbed
queries and the latent cache; agreement with the definition (original queries against keys
rebuilt from the latent cache) is reported."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import sparse_attention_indexer_02_amd as idx
from gpu_util import dev, say
from parity import check_selection

pytestmark = pytest.mark.gpu


def rne_bits_to_value(bits):
    return oracle.bf16_bits_to_f64(bits)


def check_absorbed(prob, got_bits, rows=None):
    """Every element of the GPU's absorbed queries lies between the bf16 roundings of
    exact - bound and exact + bound; returns the fraction equal to the oracle's rounding."""
    q = prob.q if rows is None else prob.q[rows]
    a = oracle.absorb_queries(q, prob.q_dtype, prob.wk)
    g = got_bits if rows is None else got_bits[rows]
    lo = rne_bits_to_value(oracle.f64_to_bf16_bits_rne(a["exact"] - a["bound"]))
    hi = rne_bits_to_value(oracle.f64_to_bf16_bits_rne(a["exact"] + a["bound"]))
    gv = rne_bits_to_value(g)
    bad = ~((gv >= lo) & (gv <= hi))
    assert not bad.any(), f"{bad.sum()} absorbed elements outside the rounding band"
    return float((g == a["bits"]).mean())


def run_latent(prob, k):
    t = dev(prob)
    ql = idx.absorb_queries(t["q"], t["wk"])
    oi, osc = idx.score_topk(ql, t["k"], t["w"], t["q_pos"], topk=k, k_len=t["k_len"], k_scale=t["k_scale"])
    torch.cuda.synchronize()
    qb = ql.view(torch.int16).cpu().numpy().view(np.uint16)
    return qb, oi.cpu().numpy(), osc.cpu().numpy()


def check_rows(prob, qb, k, gi, gs, rows, name):
    lp = oracle.latent_problem(prob, qb)
    inp = oracle.Inputs(lp)
    diff = tot = 0
    for b, t in rows:
        r = oracle.dense_row(inp, b, t, k)
        check_selection(gi[b, t], gs[b, t], r["universe"], r["all_scores"], r["magnitude"], k, lp.D,
                        ctx=f"{name} b{b} t{t}", oracle_sel=r["ids"])
        d = oracle.latent_definition_row(prob, b, t, k)
        sel = gi[b, t][gi[b, t] >= 0]
        diff += len(np.setdiff1d(d["ids"], sel))
        tot += len(d["ids"])
    say(f"{name}: recall of the definition's top-k (keys rebuilt from the latent cache) "
        f"{1 - diff / max(1, tot):.4f} over {len(rows)} rows")


@pytest.mark.parametrize("D,Dc", [(128, 64), (128, 128), (64, 32), (32, 64), (128, 32)])
def test_absorbed_queries_within_rounding_band(D, Dc):
    p = W.make_latent(2, 37, 50, H=7, D=D, Dc=Dc, seed=D + Dc)      # 518 rows: ragged tiles
    say(f"case absorb D={D} Dc={Dc} rows=2x37x7")
    t = dev(p)
    ql = idx.absorb_queries(t["q"], t["wk"])
    torch.cuda.synchronize()
    frac = check_absorbed(p, ql.view(torch.int16).cpu().numpy().view(np.uint16))
    say(f"absorb D={D} Dc={Dc}: {frac:.5f} equal to the oracle's rounding")
    assert frac > 0.99


def test_latent_prefill_all_rows():
    p = W.make_latent(1, 700, 700, H=64, D=128, Dc=64, seed=91)
    say("case latent prefill L=700 H=64 D=128 Dc=64 k=128, every row")
    qb, gi, gs = run_latent(p, 128)
    assert check_absorbed(p, qb) > 0.99
    check_rows(p, qb, 128, gi, gs, [(0, t) for t in range(p.T)], "latent-700")


@pytest.mark.parametrize("Dc", [32, 128])
def test_latent_prefill_latent_widths(Dc):
    p = W.make_latent(2, 300, 300, H=16, D=128, Dc=Dc, seed=92 + Dc)
    say(f"case latent prefill B=2 L=300 H=16 Dc={Dc} k=40")
    qb, gi, gs = run_latent(p, 40)
    check_rows(p, qb, 40, gi, gs, [(b, t) for b in range(2) for t in range(p.T)], f"latent-Dc{Dc}")


def test_latent_decode_fp8_cache():
    p = W.make_latent(4, 2, 5000, H=64, D=128, Dc=64, seed=93, k_dtype=W.FP8_E4M3, decode=True)
    p.k_len[:] = [5000, 3001, 2048, 5000]
    p.q_pos[:] = p.k_len[:, None] - 2 + np.arange(2)[None]
    say("case latent decode B=4 N=5000 T=2 FP8 latent Dc=64 k=512")
    qb, gi, gs = run_latent(p, 512)
    check_rows(p, qb, 512, gi, gs, [(b, t) for b in range(4) for t in range(2)], "latent-decode")


@pytest.mark.timeout(900)
def test_latent64k_full_size_sampled_rows():
    spec = W.WORKLOADS["latent64k"]
    p = spec["gen"](0)
    say("case latent64k full size (L=65536, H=64, D=128, Dc=64, k=2048)")
    qb, gi, gs = run_latent(p, spec["k"])
    rng = np.random.default_rng(8)
    ts = sorted(set([0, 2047, 2048, 65535] + list(rng.integers(0, 65536, 8))))
    assert check_absorbed(p, qb, rows=(slice(None), ts)) > 0.99
    check_rows(p, qb, spec["k"], gi, gs, [(0, t) for t in ts], "latent64k")
    cnt = (gi[0] >= 0).sum(-1)
    assert np.array_equal(cnt, np.minimum(spec["k"], np.arange(65536) + 1))


@pytest.mark.timeout(900)
def test_latentdec128k_full_size_sampled_sequences():
    spec = W.WORKLOADS["latentdec128k"]
    p = spec["gen"](0)
    say("case latentdec128k full size (B=32, N=131072, T=2, FP8 latent Dc=64, k=2048)")
    qb, gi, gs = run_latent(p, spec["k"])
    assert check_absorbed(p, qb) > 0.99
    check_rows(p, qb, spec["k"], gi, gs, [(b, t) for b in (0, 19, 31) for t in range(2)], "latentdec128k")
    assert ((gi >= 0).sum(-1) == spec["k"]).all()
