"""Pins for the oracle's FP8 queries (one fp32 scale per query and head, OCP E4M3FN bytes): a
hand-computed case, exact agreement with the bf16-query oracle on the same real values, and the
per-head scale acting as a factor of that head's weight."""
import numpy as np
import pytest

import oracle
import workloads as W

# E4M3FN bytes: 0x38 = 1.0, 0x40 = 2.0, 0xb8 = -1.0, 0x30 = 0.5


def _fp8_problem(q8, q_scale, k8, k_scale, w, q_pos):
    q8 = np.asarray(q8, np.uint8)[None, None]                    # one query [1,1,H,D]
    return W.Problem(q8, W.FP8_E4M3, np.asarray(k8, np.uint8)[None], W.FP8_E4M3,
                     np.asarray(k_scale, np.float32)[None], np.asarray(w, np.float32)[None, None],
                     np.array([[q_pos]], np.int32), np.array([len(k8)], np.int32),
                     q_scale=np.asarray(q_scale, np.float32)[None, None])


def test_hand_case():
    # H=1, D=2: query bytes (1.0, 2.0) with scale 0.25 -> (0.25, 0.5); w = 2
    #   key (1, 1) * 2  -> (2, 2):   dot 0.5 + 1.0  = 1.5  -> score 3.0
    #   key (-1, 1) * 1 -> (-1, 1):  dot -0.25 + 0.5 = 0.25 -> score 0.5
    #   key (-1, -1)    -> dot -0.75 -> ReLU 0 -> score 0.0
    #   key (0.5, 2) * 4 -> (2, 8):  dot 0.5 + 4.0 = 4.5 -> score 9.0
    p = _fp8_problem([[0x38, 0x40]], [0.25], [[0x38, 0x38], [0xb8, 0x38], [0xb8, 0xb8], [0x30, 0x40]],
                     [2.0, 1.0, 1.0, 4.0], [2.0], 3)
    r = oracle.dense_row(oracle.Inputs(p), 0, 0, 4)
    assert r["all_scores"].tolist() == [3.0, 0.5, 0.0, 9.0]
    assert r["ids"].tolist() == [3, 0, 1, 2]


def _finite_e4m3(rng, shape):
    b = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((b & 0x7F) == 0x7F, 0x38, b).astype(np.uint8)      # no NaN codes


def test_unit_scales_equal_bf16_queries():
    # every E4M3 value is a bf16 value: with unit query scales the FP8 query rows equal the
    # bf16-query rows of the same real values exactly
    rng = np.random.default_rng(11)
    p8 = W.make_prefill(96, 4, 32, seed=12, q_dtype=W.FP8_E4M3, k_dtype=W.FP8_E4M3)
    p8.q = _finite_e4m3(rng, p8.q.shape)
    p8.q_scale = np.ones_like(p8.q_scale)
    vals = oracle.e4m3fn_bits_to_f64(p8.q).astype(np.float32)
    qb = oracle.f32_to_bf16_bits_rne(vals).reshape(p8.q.shape)
    assert (oracle.bf16_bits_to_f64(qb) == oracle.e4m3fn_bits_to_f64(p8.q)).all()
    pb = W.Problem(qb, W.BF16, p8.k, p8.k_dtype, p8.k_scale, p8.w, p8.q_pos, p8.k_len)
    i8, i16 = oracle.Inputs(p8), oracle.Inputs(pb)
    for t in (0, 1, 31, 95):
        a, b = oracle.dense_row(i8, 0, t, 16), oracle.dense_row(i16, 0, t, 16)
        assert np.array_equal(a["all_scores"], b["all_scores"])
        assert np.array_equal(a["ids"], b["ids"])


def test_query_scale_is_a_head_weight_factor():
    # w_h ReLU(c_h x_h) = (c_h w_h) ReLU(x_h) for c_h >= 0
    rng = np.random.default_rng(13)
    p = W.make_prefill(64, 8, 64, seed=14, q_dtype=W.FP8_E4M3, k_dtype=W.FP8_E4M3)
    c = rng.uniform(0.01, 4.0, size=p.q_scale.shape).astype(np.float32)
    pa = W.Problem(p.q, p.q_dtype, p.k, p.k_dtype, p.k_scale, p.w, p.q_pos, p.k_len, q_scale=c)
    pb = W.Problem(p.q, p.q_dtype, p.k, p.k_dtype, p.k_scale,
                   (p.w.astype(np.float64) * c).astype(np.float64), p.q_pos, p.k_len,
                   q_scale=np.ones_like(c))
    ia, ib = oracle.Inputs(pa), oracle.Inputs(pb)
    ib.w = p.w.astype(np.float64) * c.astype(np.float64)             # exact products in fp64
    for t in (5, 40, 63):
        a, b = oracle.dense_row(ia, 0, t, 8), oracle.dense_row(ib, 0, t, 8)
        np.testing.assert_allclose(a["all_scores"], b["all_scores"], rtol=1e-12, atol=1e-12)


def test_generator_quantises_per_query_and_head():
    p = W.make_prefill(32, 4, 64, seed=15, q_dtype=W.FP8_E4M3, k_dtype=W.FP8_E4M3)
    q = oracle.e4m3fn_bits_to_f64(p.q)
    assert p.q_scale.shape == (1, 32, 4) and (p.q_scale > 0).all()
    assert np.abs(q).max() <= 448.0 and (np.abs(q).max(-1) > 200.0).all()   # amax maps near 448


def test_proxy_of_fp8_queries_is_refused():
    p = W.make_prefill(16, 2, 32, seed=16, q_dtype=W.FP8_E4M3, k_dtype=W.FP8_E4M3)
    with pytest.raises(ValueError):
        oracle.proxy_query(p, 0, 0, 4)
