"""Pins for the oracle's decoder building blocks: closed forms, textbook special cases and
library routines, chosen so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one of them."""

import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle as O


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.normal(size=64)
    y = O.rmsnorm(x, np.ones(64), 0.0)
    assert abs(np.sqrt(np.mean(y ** 2)) - 1.0) < 1e-12
    assert np.allclose(O.rmsnorm(7.5 * x, np.ones(64), 0.0), y, atol=1e-12)
    w = rng.normal(size=64)
    assert np.allclose(O.rmsnorm(x, w, 0.0), y * w, atol=1e-12)
    # eps enters under the root: a zero vector stays zero, a tiny vector is damped
    assert np.all(O.rmsnorm(np.zeros(4), np.ones(4), 1e-6) == 0)
    small = np.full(4, 1e-3)
    assert np.allclose(O.rmsnorm(small, np.ones(4), 1e-6), small / math.sqrt(1e-6 + 1e-6))


def test_silu_matches_library_logistic():
    x = np.linspace(-20, 20, 401)
    assert np.allclose(O.silu(x), x * expit(x), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_rope_closed_forms():
    theta = 10000.0
    # hd = 2: one pair rotated by pos radians (theta^0 = 1)
    for pos in (0, 1, 3, 17):
        r = O.rope(np.array([[1.0, 0.0]]), pos, theta)[0]
        assert np.allclose(r, [math.cos(pos), math.sin(pos)], atol=1e-14)
        r = O.rope(np.array([[0.0, 1.0]]), pos, theta)[0]
        assert np.allclose(r, [-math.sin(pos), math.cos(pos)], atol=1e-14)
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 64))
    assert np.array_equal(O.rope(x, 0, theta), x)
    for pos in (1, 100, 8191):
        assert np.allclose(np.linalg.norm(O.rope(x, pos, theta), axis=-1), np.linalg.norm(x, axis=-1))
    # pair i of hd=8 rotates at frequency theta^(-2i/8): check pair 1 (elements 1 and 5)
    e = np.zeros((1, 8)); e[0, 1] = 1.0
    r = O.rope(e, 5, theta)[0]
    ang = 5 * theta ** (-2 * 1 / 8)
    assert np.isclose(r[1], math.cos(ang)) and np.isclose(r[5], math.sin(ang))
    # relative position: <R(p)q, R(p')k> depends on p - p' only
    q, k = rng.normal(size=(1, 64)), rng.normal(size=(1, 64))
    a = float(O.rope(q, 9, theta)[0] @ O.rope(k, 4, theta)[0])
    b = float(O.rope(q, 105, theta)[0] @ O.rope(k, 100, theta)[0])
    assert abs(a - b) < 1e-10


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    hd = 16
    q = rng.normal(size=(4, hd))
    # single key: output is that key's value for every head
    K1, V1 = rng.normal(size=(2, 1, hd)), rng.normal(size=(2, 1, hd))
    o = O.attention(q, K1, V1)
    assert np.allclose(o[0], V1[0, 0]) and np.allclose(o[3], V1[1, 0])
    # all keys equal: uniform weights, output is the mean value
    K = np.repeat(rng.normal(size=(2, 1, hd)), 5, axis=1)
    V = rng.normal(size=(2, 5, hd))
    o = O.attention(q, K, V)
    assert np.allclose(o[1], V[0].mean(0)) and np.allclose(o[2], V[1].mean(0))
    # two keys: softmax of scaled scores (library softmax), with the GQA head mapping h -> h // 2
    K = rng.normal(size=(2, 2, hd))
    V = rng.normal(size=(2, 2, hd))
    o = O.attention(q, K, V)
    for h in range(4):
        g = h // 2
        s = np.array([q[h] @ K[g, 0], q[h] @ K[g, 1]]) / math.sqrt(hd)
        p = softmax(s)
        assert np.allclose(o[h], p[0] * V[g, 0] + p[1] * V[g, 1])
    # GQA equals multi-head attention with each KV head repeated for its group
    K = rng.normal(size=(2, 7, hd)); V = rng.normal(size=(2, 7, hd))
    mha = O.attention(q, np.repeat(K, 2, axis=0), np.repeat(V, 2, axis=0))
    assert np.allclose(O.attention(q, K, V), mha)
    # large score offsets do not overflow (max subtracted)
    o = O.attention(q * 1e3, K, V)
    assert np.all(np.isfinite(o))


def test_dense_ffn_closed_form():
    # 1-dim FFN: wd * silu(wg*b) * (wu*b)
    wg, wu, wd = np.array([[2.0]]), np.array([[3.0]]), np.array([[0.5]])
    b = np.array([1.5])
    expect = 0.5 * (3.0 / (1 + math.exp(-3.0))) * 4.5
    assert np.isclose(O.dense_ffn(wg, wu, wd, b)[0], expect)
    # transposition check: non-square shapes only multiply one way
    rng = np.random.default_rng(3)
    d, F = 5, 7
    Wg, Wu, Wd = rng.normal(size=(F, d)), rng.normal(size=(F, d)), rng.normal(size=(d, F))
    b = rng.normal(size=d)
    y = O.dense_ffn(Wg, Wu, Wd, b)
    ref = sum(Wd[:, f] * (Wg[f] @ b) * expit(Wg[f] @ b) * (Wu[f] @ b) for f in range(F))
    assert np.allclose(y, ref)


def test_moe_routing_special_cases():
    from workloads import ModelConfig
    d = 6
    # all router logits equal: experts 0..7, weights 1/8 each
    router = np.zeros((16, d))
    sel, w = O.moe_route(router, np.ones(d), 8)
    assert list(sel) == list(range(8)) and np.allclose(w, 1 / 8)
    # distinct logits: the top-2 by value, weights = softmax of their logits
    router = np.zeros((5, d)); router[:, 0] = [0.1, 2.0, -1.0, 1.5, 0.3]
    sel, w = O.moe_route(router, np.eye(d)[0], 2)
    assert list(sel) == [1, 3] and np.allclose(w, softmax([2.0, 1.5]))
    # one expert, top-1, zero shared FFN == a dense FFN with the expert's weights
    rng = np.random.default_rng(4)
    cfg = ModelConfig(name="m", n_layers=1, d_model=d, n_q_heads=1, n_kv_heads=1, head_dim=2,
                      ffn_dim=0, vocab=4, n_experts=1, top_k=1, expert_ffn=3, shared_ffn=2)
    lw = {"router": rng.normal(size=(1, d)), "exp_wg": rng.normal(size=(1, 3, d)),
          "exp_wu": rng.normal(size=(1, 3, d)), "exp_wd": rng.normal(size=(1, d, 3)),
          "sh_wg": np.zeros((2, d)), "sh_wu": np.zeros((2, d)), "sh_wd": np.zeros((d, 2))}
    b = rng.normal(size=d)
    assert np.allclose(O.moe_ffn(lw, cfg, b), O.dense_ffn(lw["exp_wg"][0], lw["exp_wu"][0], lw["exp_wd"][0], b))


def test_moe_route_margin_and_convex_mixture():
    d = 6
    router = np.zeros((5, d)); router[:, 0] = [0.1, 2.0, -1.0, 1.5, 0.3]
    assert np.isclose(O.moe_route_margin(router, np.eye(d)[0], 2), 1.5 - 0.3)
    assert O.moe_route_margin(router, np.eye(d)[0], 5) == np.inf
    # identical experts: the routing weights sum to one, so the mixture equals one expert's FFN
    # (plus the shared FFN) whatever the router says
    from workloads import ModelConfig
    rng = np.random.default_rng(9)
    cfg = ModelConfig(name="m", n_layers=1, d_model=d, n_q_heads=1, n_kv_heads=1, head_dim=2,
                      ffn_dim=0, vocab=4, n_experts=5, top_k=3, expert_ffn=4, shared_ffn=3)
    wg, wu, wd = rng.normal(size=(4, d)), rng.normal(size=(4, d)), rng.normal(size=(d, 4))
    sg, su, sd = rng.normal(size=(3, d)), rng.normal(size=(3, d)), rng.normal(size=(d, 3))
    lw = {"router": rng.normal(size=(5, d)), "exp_wg": np.stack([wg] * 5),
          "exp_wu": np.stack([wu] * 5), "exp_wd": np.stack([wd] * 5),
          "sh_wg": sg, "sh_wu": su, "sh_wd": sd}
    b = rng.normal(size=d)
    tr = []
    y = O.moe_ffn(lw, cfg, b, trace=tr)
    assert np.allclose(y, O.dense_ffn(wg, wu, wd, b) + O.dense_ffn(sg, su, sd, b))
    assert len(tr) == 1 and tr[0] == O.moe_route_margin(lw["router"], b, 3)


def test_argmax_first_ties_and_nan():
    assert O.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert O.argmax_first(np.array([5.0, 5.0])) == 0
    with pytest.raises(FloatingPointError):
        O.argmax_first(np.array([1.0, np.nan]))
    assert O.top2_margin(np.array([0.5, 2.0, 1.25])) == 0.75
