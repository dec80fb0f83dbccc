"""Pins for the oracle's decoder, acceptance, drafter head and speculative loop.

What fixes the expected values here: the pages' invariants (speculative output equals the
target's own greedy output; each step yields between 1 and K+1 tokens; all-correct drafts
yield K+1 and all-wrong drafts yield 1), an independent matrix-form causal forward, brute
force over every draft tuple on a micro model, and special cases of the clustered head."""

import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O
from workloads import ModelConfig, drafter_weights, preset, prompt_tokens, target_weights

GOLD = os.path.join(os.path.dirname(__file__), "golden")

MICRO = ModelConfig(name="micro", n_layers=2, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8,
                    ffn_dim=32, vocab=16, d_layers=1, d_dim=8, d_ffn=32, n_centroids=4,
                    dtype="f32", init="normal", seed=5, weight_std=0.5, norm_jitter=0.2,
                    prompt_len=5, gen_tokens=12, draft_k=2)

MICRO_MOE = MICRO.replace(name="micro-moe", ffn_dim=0, n_experts=4, top_k=2, expert_ffn=8,
                          shared_ffn=8, seed=6)


def build(cfg):
    W = O.as_f64(target_weights(cfg))
    DW = O.as_f64(drafter_weights(cfg))
    return W, DW


def start_state(cfg, W, extra=16):
    prompt = prompt_tokens(cfg)[0]
    cache = O.KVCache.empty(cfg, cfg.prompt_len + cfg.gen_tokens + extra)
    t0, hid, length = O.prefill(W, cfg, cache, prompt)
    return cache, t0, hid, length


def matrix_forward(W, cfg, toks):
    """Independent causal forward over a whole sequence in matrix form.  RoPE is written as a
    complex rotation of (x_i + i x_{i+hd/2}); attention uses a masked score matrix."""
    n, hd = len(toks), cfg.head_dim
    half = hd // 2
    X = W["embed"][np.array(toks)]

    def rms(A, w):
        return A / np.sqrt((A ** 2).mean(-1, keepdims=True) + cfg.rms_eps) * w

    def rot(A):  # A: [n][H][hd]
        out = np.empty_like(A)
        for p in range(n):
            for i in range(half):
                f = cmath.exp(1j * p * cfg.rope_theta ** (-2.0 * i / hd))
                zc = (A[p, :, i] + 1j * A[p, :, i + half]) * f
                out[p, :, i], out[p, :, i + half] = zc.real, zc.imag
        return out

    mask = np.triu(np.full((n, n), -np.inf), 1)
    for lw in W["layers"]:
        A = rms(X, lw["attn_norm"])
        Q = rot((A @ lw["wq"].T).reshape(n, cfg.n_q_heads, hd))
        Kx = rot((A @ lw["wk"].T).reshape(n, cfg.n_kv_heads, hd))
        Vx = (A @ lw["wv"].T).reshape(n, cfg.n_kv_heads, hd)
        Oh = np.empty_like(Q)
        for h in range(cfg.n_q_heads):
            g = h // cfg.group
            S = Q[:, h] @ Kx[:, g].T / math.sqrt(hd) + mask
            Oh[:, h] = softmax(S, axis=-1) @ Vx[:, g]
        X = X + Oh.reshape(n, -1) @ lw["wo"].T
        B = rms(X, lw["ffn_norm"])
        if cfg.is_moe:
            X = X + np.stack([O.moe_ffn(lw, cfg, B[p]) for p in range(n)])
        else:
            G = B @ lw["wg"].T
            X = X + (G / (1 + np.exp(-G)) * (B @ lw["wu"].T)) @ lw["wd"].T
    return rms(X, W["final_norm"]) @ W["embed"].T, X


@pytest.mark.parametrize("cfg", [MICRO, MICRO_MOE], ids=["dense", "moe"])
def test_incremental_decode_equals_matrix_forward(cfg):
    W, _ = build(cfg)
    toks = list(prompt_tokens(cfg)[0]) + [3, 9, 1]
    cache = O.KVCache.empty(cfg, 32)
    rows = [O.target_row(W, cfg, cache, t, p) for p, t in enumerate(toks)]
    L_ref, H_ref = matrix_forward(W, cfg, toks)
    for p, (lg, hd) in enumerate(rows):
        assert np.allclose(lg, L_ref[p], rtol=1e-10, atol=1e-10)
        assert np.allclose(hd, H_ref[p], rtol=1e-10, atol=1e-10)


def test_causality_and_k0_verify_is_decode():
    W, _ = build(MICRO)
    cache, t0, hid, length = start_state(MICRO, W)
    c1, c2 = cache.copy(), cache.copy()
    G, H, Ls = O.verify(W, MICRO, c1, length, [t0])
    lg, hd = O.target_row(W, MICRO, c2, t0, length)
    assert np.array_equal(Ls[0], lg) and np.array_equal(H[0], hd) and G[0] == O.argmax_first(lg)
    # later rows never change earlier rows
    a = O.verify(W, MICRO, cache.copy(), length, [t0, 1, 2])
    b = O.verify(W, MICRO, cache.copy(), length, [t0, 1, 7])
    assert np.array_equal(a[2][0], b[2][0]) and np.array_equal(a[2][1], b[2][1])
    assert not np.array_equal(a[2][2], b[2][2])


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_accept_closed_form_all_patterns(K):
    rng = np.random.default_rng(K)
    for pattern in itertools.product([0, 1], repeat=K):
        G = list(rng.integers(0, 100, size=K + 1))
        T = [int(rng.integers(0, 100))]
        for j in range(K):
            T.append(int(G[j]) if pattern[j] else int(G[j]) + 100)
        m_expect = next((j for j, bit in enumerate(pattern) if not bit), K)
        m, out, nxt = O.accept(T, G)
        assert m == m_expect
        assert out == [int(g) for g in G[:m]] + [int(G[m])]
        assert len(out) == m + 1 and 1 <= len(out) <= K + 1
        assert nxt == int(G[m])


def test_brute_force_every_draft_tuple_micro():
    """For every tuple in V^K, one draft-verify-accept step emits exactly the greedy prefix."""
    cfg = MICRO
    W, _ = build(cfg)
    cache, t0, hid, length = start_state(cfg, W)
    K = 2
    greedy = O.greedy_generate(W, cfg, cache.copy(), t0, length, K + 2)  # pos length .. length+K+1
    for tup in itertools.product(range(cfg.vocab), repeat=K):
        T = [t0] + list(tup)
        G, H, _ = O.verify(W, cfg, cache.copy(), length, T)
        m, out, nxt = O.accept(T, G)
        m_expect = 0
        while m_expect < K and tup[m_expect] == greedy[m_expect + 1]:
            m_expect += 1
        assert m == m_expect
        assert out == greedy[1 : m + 2]


def _tiny_run(p, forced_wrong=False, head_mode="clustered", k_c=1, poison=False, cfg=None):
    cfg = cfg or preset("tiny")
    W, DW = build(cfg)
    cache, t0, hid, length = start_state(cfg, W)
    K, n = cfg.draft_k, cfg.gen_tokens
    greedy, margins = O.greedy_generate(W, cfg, cache.copy(), t0, length, n + K + 1,
                                         record_margins=True)
    gseq = np.zeros(length + len(greedy), dtype=np.int64)
    gseq[length:] = greedy
    toks, st = O.spec_generate(W, DW, cfg, cache, t0, hid, length, n, K, greedy_seq=gseq, p=p,
                               seed=cfg.inject_seed, head_mode=head_mode, k_c=k_c,
                               forced_wrong=forced_wrong, poison=poison)
    return toks, greedy[:n], st


@pytest.mark.parametrize("p", [0.0, 0.6, 1.0])
def test_tiny_spec_equals_greedy(p):
    toks, greedy, st = _tiny_run(p)
    assert toks == greedy
    K = preset("tiny").draft_k
    assert all(1 <= e <= K + 1 for e in st.emitted_per_step)
    assert math.isclose(st.tokens_per_pass, 1 + st.accepted / st.steps)
    if p == 1.0:
        assert all(e == K + 1 for e in st.emitted_per_step)
        assert st.steps == math.ceil((len(toks) - 1) / (K + 1))
    if p == 0.0:
        # random-init drafts essentially never hit the greedy token
        assert st.accepted <= 2


def test_tiny_forced_wrong_emits_one_per_step_and_poison_is_never_read():
    toks, greedy, st = _tiny_run(0.0, forced_wrong=True, poison=True)
    assert toks == greedy
    assert all(e == 1 for e in st.emitted_per_step)
    toks, greedy, st = _tiny_run(0.6, poison=True, head_mode="full")
    assert toks == greedy


def test_moe_spec_equals_greedy_micro():
    cfg = MICRO_MOE.replace(gen_tokens=10)
    toks, greedy, st = _tiny_run(0.6, cfg=cfg)
    assert toks == greedy


def test_clustered_head_special_cases():
    rng = np.random.default_rng(7)
    V, D, Nc = 64, 8, 8
    S = V // Nc
    for trial in range(50):
        table = rng.normal(size=(V, D))
        perm = rng.permutation(V)
        s = rng.normal(size=D)
        w = O.head_full(table, s)
        if trial % 2 == 0:
            # exact tie at the maximum with a higher vocab id: the lower id (w) must still win
            dup = V - 1 if w != V - 1 else 0
            table[dup] = table[w]
            w = min(w, dup)
        C = table[perm].reshape(Nc, S, D).mean(1)
        full = O.head_full(table, s)
        assert full == w
        assert O.head_clustered(table, C, perm, s, Nc) == full
        # one cluster holding every token is the full head
        assert O.head_clustered(table, table.mean(0, keepdims=True), rng.permutation(V), s, 1) == full
        # once the winner's cluster is among the selected ones the clustered head returns it
        z = C @ s
        winner_cluster = int(np.where(perm == full)[0][0]) // S
        rank = sorted(range(Nc), key=lambda c: (-z[c], c)).index(winner_cluster)
        for k_c in range(rank + 1, Nc + 1):
            assert O.head_clustered(table, C, perm, s, k_c) == full
        # with k_c = 1 the result is a member of the best-scoring cluster
        top = sorted(range(Nc), key=lambda c: (-z[c], c))[0]
        assert O.head_clustered(table, C, perm, s, 1) in set(perm[top * S:(top + 1) * S])


def test_drafter_reads_only_committed_cache_and_is_prefix_consistent():
    cfg = preset("tiny")
    W, DW = build(cfg)
    cache, t0, hid, length = start_state(cfg, W)
    d3 = O.draft(DW, cfg, cache, hid, t0, length, 3)
    poisoned = cache.copy()
    for l in range(cfg.n_layers):
        poisoned.K[l][:, length:] = np.nan
        poisoned.V[l][:, length:] = np.nan
    assert O.draft(DW, cfg, poisoned, hid, t0, length, 3) == d3
    assert O.draft(DW, cfg, cache, hid, t0, length, 2) == d3[:2]
    assert O.draft(DW, cfg, cache, hid, t0, length, 3, head_mode="clustered",
                   k_c=cfg.n_centroids) == O.draft(DW, cfg, cache, hid, t0, length, 3, head_mode="full")


def test_page_accounting_is_consistent_with_the_step_rule():
    g = json.load(open(os.path.join(GOLD, "llamacpp_accounting.json")))
    passes = g["accepted"] / (g["tokens_per_pass"] - 1.0)  # each pass emits accepted + 1
    assert 1.0 <= g["proposed"] / passes <= g["draft_n_max"] + 1e-9
    assert 1.0 <= g["tokens_per_pass"] <= g["draft_n_max"] + 1
    # i.i.d. per-slot acceptance fitted to the tokens-per-pass figure reproduces the acceptance ratio
    p = next(x / 1000 for x in range(1000) if 1 + x / 1000 + (x / 1000) ** 2 >= g["tokens_per_pass"])
    assert abs(p - 0.89) < 0.01
