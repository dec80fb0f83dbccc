"""Pins for the oracle's token trees (draft_tree, verify_tree, accept_tree, commit_tree,
spec_generate_tree).

What fixes the expected values: a one-branch tree is a linear draft, so it must reproduce the
linear functions exactly (drafts, verify rows, acceptance); speculative output with trees equals
the target's own greedy output (the pages' invariant: drafts only change speed); a tree whose
nodes all hold the target's greedy tokens emits depth + 1 tokens per step; constructed trees where
only a later branch holds the greedy continuation accept along that branch; the committed cache
equals plain decoding's."""

import numpy as np
import pytest

import oracle as O
from workloads import ModelConfig, drafter_weights, preset, prompt_tokens, target_weights

MICRO = ModelConfig(name="micro", n_layers=2, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8,
                    ffn_dim=32, vocab=16, d_layers=1, d_dim=8, d_ffn=32, n_centroids=4,
                    dtype="f32", init="normal", seed=5, weight_std=0.5, norm_jitter=0.2,
                    prompt_len=5, gen_tokens=12, draft_k=2)


def setup(cfg, extra=24):
    W = O.as_f64(target_weights(cfg))
    DW = O.as_f64(drafter_weights(cfg))
    prompt = prompt_tokens(cfg)[0]
    cache = O.KVCache.empty(cfg, cfg.prompt_len + cfg.gen_tokens + extra)
    t0, hid, length = O.prefill(W, cfg, cache, prompt)
    return W, DW, cache, t0, hid, length


def test_tree_shape():
    par = O.tree_parents(3, 2)
    assert par == [-1, 0, 0, 0, 1, 2, 3]
    assert O.tree_path(par, 5) == [0, 2, 5]
    assert O.tree_parents(1, 4) == [-1, 0, 1, 2, 3]


@pytest.mark.parametrize("mode,k_c", [("clustered", 1), ("clustered", 2), ("full", 1)])
def test_one_branch_tree_is_the_linear_draft(mode, k_c):
    cfg = preset("tiny")
    W, DW, cache, t0, hid, length = setup(cfg)
    lin = O.draft(DW, cfg, cache, hid, t0, length, 3, head_mode=mode, k_c=k_c)
    tree = O.draft_tree(DW, cfg, cache, hid, t0, length, 1, 3, head_mode=mode, k_c=k_c)
    assert tree == [t0] + lin
    par = O.tree_parents(1, 3)
    G, H, L = O.verify(W, cfg, cache.copy(), length, tree)
    Gt, Ht, Lt = O.verify_tree(W, cfg, cache, length, tree, par)
    assert G == Gt
    assert all(np.array_equal(a, b) for a, b in zip(H, Ht))
    assert all(np.array_equal(a, b) for a, b in zip(L, Lt))
    m, out, nxt = O.accept(tree, G)
    mt, outt, nxtt, nodes = O.accept_tree(tree, par, Gt)
    assert (m, out, nxt) == (mt, outt, nxtt) and nodes == list(range(1, m + 1))


def test_head_top_ranks_by_score_then_lower_id():
    rng = np.random.default_rng(4)
    V, D, Nc = 32, 6, 4
    table = rng.normal(size=(V, D))
    table[7] = table[20]  # an exact tie: 7 must come before 20
    perm = rng.permutation(V)
    S = V // Nc
    DW = {"table": table, "perm": perm, "centroids": table[perm].reshape(Nc, S, D).mean(1)}
    s = table[20] + 0.0
    top = O.head_top(DW, s, 5, "full")
    sc = table @ s
    want = sorted(range(V), key=lambda t: (-sc[t], t))[:5]
    assert top == want and top.index(7) < top.index(20)
    assert O.head_top(DW, s, 1, "full") == [O.head_full(table, s)]
    assert O.head_top(DW, s, 1, "clustered", 2) == [O.head_clustered(table, DW["centroids"], perm, s, 2)]


def test_later_branch_with_the_greedy_path_is_accepted():
    cfg = MICRO
    W, DW, cache, t0, hid, length = setup(cfg)
    greedy = O.greedy_generate(W, cfg, cache.copy(), t0, length, 6)
    width, depth = 3, 3
    par = O.tree_parents(width, depth)
    # branch 2 holds the greedy continuation, branches 0 and 1 a wrong first token
    T = [t0]
    for j in range(1, depth + 1):
        for k in range(width):
            T.append(greedy[j] if k == 2 else (greedy[j] + 1 + k) % cfg.vocab)
    G, H, _ = O.verify_tree(W, cfg, cache, length, T, par)
    m, out, nxt, nodes = O.accept_tree(T, par, G)
    assert m == depth and out == greedy[1:depth + 2] and nxt == greedy[depth + 1]
    assert nodes == [1 + width * (j - 1) + 2 for j in range(1, depth + 1)]
    # committing leaves exactly plain decoding's cache and hidden state
    c_tree, c_plain = cache.copy(), cache.copy()
    new_len, h = O.commit_tree(W, cfg, c_tree, length, T, nodes, H)
    lg = hd = None
    for j, tok in enumerate(greedy[:depth + 1]):
        lg, hd = O.target_row(W, cfg, c_plain, tok, length + j)
    assert new_len == length + depth + 1 and np.array_equal(h, hd)
    for l in range(cfg.n_layers):
        assert np.array_equal(c_tree.K[l][:, :new_len], c_plain.K[l][:, :new_len])
        assert np.array_equal(c_tree.V[l][:, :new_len], c_plain.V[l][:, :new_len])


def test_random_trees_emit_the_greedy_prefix():
    cfg = MICRO
    W, DW, cache, t0, hid, length = setup(cfg)
    greedy = O.greedy_generate(W, cfg, cache.copy(), t0, length, 6)
    rng = np.random.default_rng(9)
    par = O.tree_parents(2, 2)
    for _ in range(60):
        # each node holds its greedy token or a random one
        T = [t0]
        for i in range(1, len(par)):
            dpt = len(O.tree_path(par, i)) - 1
            T.append(greedy[dpt] if rng.random() < 0.6 else int(rng.integers(cfg.vocab)))
        G, _, _ = O.verify_tree(W, cfg, cache, length, T, par)
        m, out, nxt, nodes = O.accept_tree(T, par, G)
        assert out == greedy[1:m + 2]
        # m is the longest greedy-agreeing root path (the target agrees exactly where the greedy
        # token sits, since every node on an agreeing path extends the greedy prefix)
        best = 0
        for i in range(1, len(par)):
            path = O.tree_path(par, i)
            if all(T[n] == greedy[j] for j, n in enumerate(path) if j > 0):
                best = max(best, len(path) - 1)
        assert m == best


@pytest.mark.parametrize("width,p", [(1, 0.6), (2, 0.6), (3, 0.0), (3, 1.0)])
def test_tree_spec_equals_greedy(width, p):
    cfg = preset("tiny", gen_tokens=24)
    W, DW, cache, t0, hid, length = setup(cfg, extra=32)
    depth, n = 3, cfg.gen_tokens
    greedy = O.greedy_generate(W, cfg, cache.copy(), t0, length, n + depth + 2)
    gseq = np.zeros(length + len(greedy), dtype=np.int64)
    gseq[length:] = greedy
    toks, st = O.spec_generate_tree(W, DW, cfg, cache, t0, hid, length, n, width, depth,
                                    greedy_seq=gseq, p=p, seed=cfg.inject_seed)
    assert toks == greedy[:n]
    assert all(1 <= e <= depth + 1 for e in st.emitted_per_step)
    if p == 1.0:
        assert all(e == depth + 1 for e in st.emitted_per_step[:-1])


def test_binding_tree_shape_is_the_oracle_shape():
    from speculative_decoding_03_amd.engine import tree_parents
    for w in (1, 2, 3, 4):
        for d in (1, 2, 3, 5):
            assert tree_parents(w, d) == O.tree_parents(w, d)
