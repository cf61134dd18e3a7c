"""Pins for the oracle's absorbed-query scoring of a shared latent cache ("LatentIndex: Cross-Layer
Sharing with Layer-Specific Selection for Sparse Attention", abstract): the direct binary64 ->
bfloat16 rounding (ties, a case where rounding through fp32 first would differ, and agreement with
torch's conversion wherever the value is exact in fp32), a hand-computed absorption, the identity
decoder, the scoring identity with keys rebuilt from the latent cache, and the error bound."""
import numpy as np
import torch

import oracle
import workloads as W


def bf16_value(bits):
    return oracle.bf16_bits_to_f64(np.asarray(bits, np.uint16))


def test_f64_to_bf16_ties_and_single_rounding():
    x = np.array([1.0 + 2.0 ** -8,                    # halfway 1 | 1+2^-7: to even, 1
                  1.0 + 3 * 2.0 ** -8,                # halfway 1+2^-7 | 1+2^-6: to even, 1+2^-6
                  1.0 + 2.0 ** -8 + 2.0 ** -40,       # just above halfway: up (through fp32: a tie, down)
                  -(1.0 + 2.0 ** -8 + 2.0 ** -40),
                  0.0, -0.0, 3.0, 2.0 ** -130, 1.5 * 2.0 ** -133])
    got = bf16_value(oracle.f64_to_bf16_bits_rne(x))
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 0.0, 0.0, 3.0,
                     2.0 ** -130, 2.0 * 2.0 ** -133])
    assert np.array_equal(got, want)
    assert oracle.f64_to_bf16_bits_rne(np.array([-0.0]))[0] == 0x8000


def test_f64_to_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits_rne(x.astype(np.float64)), ref)


def test_absorb_hand_case():
    # q = [1, 2] (H = 1, D = 2); decoder rows [1, 0], [1, 1], [0, 3] (Dc = 3): Wk q = [1, 3, 6]
    q = W.f32_to_bf16_bits(np.array([[[1.0, 2.0]]], np.float32))
    wk = W.f32_to_bf16_bits(np.array([[1.0, 0.0], [1.0, 1.0], [0.0, 3.0]], np.float32))
    a = oracle.absorb_queries(q, oracle.BF16, wk)
    assert a["bits"].shape == (1, 1, 3)
    assert np.array_equal(bf16_value(a["bits"])[0, 0], [1.0, 3.0, 6.0])
    assert np.allclose(a["bound"][0, 0], np.array([1.0, 3.0, 6.0]) * 2 * 2.0 ** -24)
    # fp32 queries take the same path
    a32 = oracle.absorb_queries(np.array([[[1.0, 2.0]]], np.float32), oracle.F32, wk)
    assert np.array_equal(a32["bits"], a["bits"])


def test_absorb_identity_decoder_keeps_the_queries():
    rng = np.random.default_rng(3)
    q = W.f32_to_bf16_bits(rng.standard_normal((2, 5, 4, 32)).astype(np.float32))
    eye = W.f32_to_bf16_bits(np.eye(32, dtype=np.float32))
    a = oracle.absorb_queries(q, oracle.BF16, eye)
    assert np.array_equal(a["bits"], q)
    assert np.array_equal(a["exact"], oracle.bf16_bits_to_f64(q))


def test_absorbed_scores_equal_scores_of_rebuilt_keys():
    # q . (c Wk) = (Wk q) . c: the exact absorbed queries against the latent rows give the scores
    # of the original queries against the rebuilt keys (up to float64 rounding); a decoder used
    # transposed or on the wrong side breaks this (Dc != D)
    p = W.make_latent(1, 40, 40, H=8, D=64, Dc=32, seed=5)
    a = oracle.absorb_queries(p.q, p.q_dtype, p.wk)
    lat = oracle.keys_f64(p.k[0], p.k_dtype, None)
    w = p.w[0].astype(np.float64)
    for t in (0, 17, 39):
        rdef = oracle.latent_definition_row(p, 0, t, 8)
        s_abs = oracle.index_scores(a["exact"][0, t], w[t], lat[:t + 1])
        assert np.allclose(s_abs, rdef["all_scores"], rtol=1e-12, atol=1e-12)
        assert np.array_equal(oracle.select_topk(s_abs, np.arange(t + 1), 8)[0], rdef["ids"])


def test_absorbed_bf16_queries_stay_within_their_rounding_of_the_definition():
    # the stored (rounded) absorbed queries move each dot product by at most half a bf16 unit per
    # element: |I_lat - I_def| <= sum_h |w_h| sum_j 2^-9 |q~_hj| |c_j| (relative half-unit 2^-9)
    p = W.make_latent(1, 64, 64, H=8, D=128, Dc=64, seed=6)
    a = oracle.absorb_queries(p.q, p.q_dtype, p.wk)
    assert (np.abs(bf16_value(a["bits"]) - a["exact"]) <= np.abs(a["exact"]) * 2.0 ** -8).all()
    lp = oracle.latent_problem(p, a["bits"])
    inp = oracle.Inputs(lp)
    lat = inp.keys(0)
    for t in (10, 63):
        r = oracle.dense_row(inp, 0, t, 16)
        d = oracle.latent_definition_row(p, 0, t, 16)
        qb = bf16_value(a["bits"][0, t])
        bound = (np.abs(lat[:t + 1]) @ (np.abs(qb) * 2.0 ** -8).T) @ np.abs(p.w[0, t].astype(np.float64))
        assert (np.abs(r["all_scores"] - d["all_scores"]) <= bound).all()


def test_error_bound_scales_with_the_magnitudes():
    q = W.f32_to_bf16_bits(np.array([[[1.0, -2.0, 4.0]]], np.float32))
    wk = W.f32_to_bf16_bits(np.array([[1.0, 1.0, 1.0], [-1.0, 0.5, 0.25]], np.float32))
    a = oracle.absorb_queries(q, oracle.BF16, wk)
    assert np.array_equal(a["exact"][0, 0], [3.0, -1.0])
    assert np.array_equal(a["bound"][0, 0], np.array([7.0, 3.0]) * 3 * 2.0 ** -24)
