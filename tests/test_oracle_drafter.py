"""Pins for the oracle's drafter sub-step (oracle.drafter_substep / oracle.draft).

The pages fix what the drafter reads and how it proceeds, not its numbers: it takes the target's
last hidden state and the token, cross-attends into the target's own KV cache with no cache of
its own, and proposes tokens one after another, each sub-step feeding the next ("Accelerating
Gemini Nano on Pixel with frozen multi-token prediction", sections "The 'late exit' strategy" and
"Zero-copy architecture"; "Gemma 4's MTP drafter explained", section "What is different about
Gemma 4's drafter?").  The wiring the oracle takes where the pages are silent (input
W_in [rms(h) n_h ; rms(e) n_e], query at position len + j - 1, keys [0, len) of the target's last
layer, next hidden W_back s) is pinned here by:

* hand-worked closed forms on 2-wide weights chosen so that every quantity can be written out
  (a zero query projection makes the attention the plain mean of the source layer's values; a
  2-wide head dimension has one rotary pair turning by exactly `pos` radians; zero gate weights
  remove the FFN);
* an independent drafter written with explicit loops over elements and heads, complex-number
  rotary embedding and a split input projection, compared on random micro weights;
* planted mistakes: each plausible slip (concatenation order, rotary position, source layer,
  a dropped norm weight, W_back applied to the wrong vector, the key range, the second norm) is
  written into a copy of the oracle's source, and at least one pin must fail on it."""

import cmath
import math
import os
import sys
import types

import numpy as np
import pytest

import oracle as O
from workloads import ModelConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def micro_cfg(**kw):
    base = dict(name="drafter-pin", n_layers=2, d_model=2, n_q_heads=1, n_kv_heads=1, head_dim=2,
                ffn_dim=2, vocab=4, d_layers=1, d_dim=2, d_ffn=2, n_centroids=2, dtype="f32",
                init="normal", rms_eps=0.0, rope_theta=10000.0)
    base.update(kw)
    return ModelConfig(**base)


def zero_layer(cfg):
    D, qd, F = cfg.d_dim, cfg.q_dim, cfg.d_ffn
    return {"n1": np.ones(D), "wq": np.zeros((qd, D)), "wo": np.zeros((D, qd)), "n2": np.ones(D),
            "wg": np.zeros((F, D)), "wu": np.zeros((F, D)), "wd": np.zeros((D, F))}


def drafter(cfg, w_in, layers, norm_h=(1.0, 1.0), norm_e=(1.0, 1.0), norm_f=(1.0, 1.0),
            w_back=None):
    table = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 2.0], [-1.0, -1.0]])
    perm = np.arange(4)
    return {"table": table, "perm": perm, "centroids": table.reshape(2, 2, 2).mean(1),
            "norm_h": np.array(norm_h), "norm_e": np.array(norm_e), "w_in": np.array(w_in, float),
            "layers": layers, "norm_f": np.array(norm_f),
            "w_back": np.eye(2) if w_back is None else np.array(w_back, float)}


def cache_with(cfg, cap, src_vals, other_vals, src_keys=None, other_keys=None):
    """A cache whose source layer (the last) and other layer hold the given value / key rows
    for positions [0, n); positions from n on hold NaN (dead slots)."""
    c = O.KVCache.empty(cfg, cap)
    for l in range(cfg.n_layers):
        c.K[l][:] = np.nan
        c.V[l][:] = np.nan
    for l, vals, keys in ((cfg.n_layers - 1, src_vals, src_keys), (0, other_vals, other_keys)):
        vals = np.asarray(vals, float)  # [Hkv][n][hd]
        n = vals.shape[1]
        c.V[l][:, :n] = vals
        c.K[l][:, :n] = np.zeros_like(vals) if keys is None else np.asarray(keys, float)
    return c


def unit(v):
    v = np.asarray(v, float)
    return v / math.sqrt(float(np.mean(v * v)))


# ---------------------------------------------------------------------------------------------
# The pins, each taking the oracle module so that planted mistakes can be run through them.
# ---------------------------------------------------------------------------------------------

def pin_input_wiring(O):
    """x = W_in [rms(h) n_h ; rms(e) n_e]; s = rms(x) n_f; next hidden = W_back s.  Attention and
    FFN are switched off (zero query, output and gate weights), so the final x is the input
    projection itself."""
    cfg = micro_cfg()
    cache = cache_with(cfg, 8, [[[1.0, 0.0]]], [[[0.0, 1.0]]])
    h = np.array([3.0, 1.0])
    n_h, n_e, n_f = (1.0, 2.0), (2.0, 1.0), (1.0, 3.0)
    e = np.array([1.0, 2.0])  # table row of token 2
    w_back = [[0.5, 1.0], [2.0, -1.0]]
    # the h half of the input only
    DW = drafter(cfg, [[1, 0, 0, 0], [0, 1, 0, 0]], [zero_layer(cfg)], n_h, n_e, n_f, w_back)
    tr = []
    d, hn = O.drafter_substep(DW, cfg, cache, h, 2, 1, 1, "full", 1, tr)
    x = unit(h) * np.array(n_h)
    s = unit(x) * np.array(n_f)
    assert np.allclose(tr[0], s, rtol=1e-12, atol=1e-12)
    assert np.allclose(hn, np.array(w_back) @ s, rtol=1e-12, atol=1e-12)
    assert d == int(np.argmax(DW["table"] @ s))
    # the token half of the input only
    DW = drafter(cfg, [[0, 0, 1, 0], [0, 0, 0, 1]], [zero_layer(cfg)], n_h, n_e, n_f, w_back)
    tr = []
    d, hn = O.drafter_substep(DW, cfg, cache, h, 2, 1, 1, "full", 1, tr)
    x = unit(e) * np.array(n_e)
    s = unit(x) * np.array(n_f)
    assert np.allclose(tr[0], s, rtol=1e-12, atol=1e-12)
    assert np.allclose(hn, np.array(w_back) @ s, rtol=1e-12, atol=1e-12)
    # both halves, mixed: x0 = rms(h) n_h + 2 rms(e) n_e elementwise
    DW = drafter(cfg, [[1, 0, 2, 0], [0, 1, 0, 2]], [zero_layer(cfg)], n_h, n_e, n_f, w_back)
    tr = []
    O.drafter_substep(DW, cfg, cache, h, 2, 1, 1, "full", 1, tr)
    x = unit(h) * np.array(n_h) + 2 * unit(e) * np.array(n_e)
    assert np.allclose(tr[0], unit(x) * np.array(n_f), rtol=1e-12, atol=1e-12)


def pin_source_layer_key_range_and_grouping(O):
    """A zero query projection makes every score 0, so each query head's output is the plain
    mean of its KV head's values over the visible keys [0, len) of the source layer (the
    target's last).  Four query heads over two KV heads: heads 0, 1 read KV head 0 and heads
    2, 3 read KV head 1.  Dead slots from len on hold NaN and must not be read."""
    cfg = micro_cfg(n_q_heads=4, n_kv_heads=2)
    length = 3
    src = [[[1.0, 0.0], [2.0, 0.0], [3.0, 0.0]],     # KV head 0: mean (2, 0)
           [[0.0, 2.0], [0.0, 4.0], [0.0, 6.0]]]     # KV head 1: mean (0, 4)
    other = [[[0.0, 9.0]] * 3, [[9.0, 0.0]] * 3]     # layer 0: different means
    cache = cache_with(cfg, 8, src, other)
    lay = zero_layer(cfg)
    # o = [o_h0 ; o_h1 ; o_h2 ; o_h3]; x += (o_h0[0] + 10 o_h1[0], o_h2[1] + 10 o_h3[1])
    wo = np.zeros((2, 8))
    wo[0, 0], wo[0, 2], wo[1, 5], wo[1, 7] = 1.0, 10.0, 1.0, 10.0
    lay["wo"] = wo
    DW = drafter(cfg, [[1, 0, 0, 0], [0, 1, 0, 0]], [lay])
    h = np.array([1.0, 1.0])
    tr = []
    O.drafter_substep(DW, cfg, cache, h, 0, length, length, "full", 1, tr)
    x = unit(h) + np.array([2.0 + 10 * 2.0, 4.0 + 10 * 4.0])
    assert np.allclose(tr[0], unit(x), rtol=1e-12, atol=1e-12)


def pin_rope_position(O):
    """One rotary pair (head size 2) turns by exactly pos radians.  With query q = (sqrt 2, 0)
    before rotation, keys (k, 0) and (-k, 0) and values (1, 0), (0, 1), the weight of the first
    key is 1 / (1 + exp(-2 k cos t)) at rotation t.  Sub-step j of a draft from length len
    queries at t = len + j - 1."""
    cfg = micro_cfg(rope_theta=12345.0)
    length, kap = 2, 1.5
    cache = cache_with(cfg, 8, [[[1.0, 0.0], [0.0, 1.0]]], [[[0.0, 0.0], [0.0, 0.0]]],
                       src_keys=[[[kap, 0.0], [-kap, 0.0]]])
    lay = zero_layer(cfg)
    lay["wq"] = np.eye(2)
    lay["wo"] = np.eye(2)
    DW = drafter(cfg, [[1, 0, 0, 0], [0, 1, 0, 0]], [lay], norm_f=(1.0, 2.0))
    h = np.array([1.0, 0.0])
    tr = []
    O.draft(DW, cfg, cache, h, 0, length, 2, head_mode="full", trace=tr)
    hh = h
    for j in (1, 2):
        x0 = unit(hh)                          # W_in picks rms(h) (n_h = 1)
        a = unit(x0)                           # n1 = 1
        q = a                                  # W_q = I
        t = length + j - 1
        qr = np.array([q[0] * math.cos(t) - q[1] * math.sin(t), q[1] * math.cos(t) + q[0] * math.sin(t)])
        s0, s1 = qr @ np.array([kap, 0.0]) / math.sqrt(2), qr @ np.array([-kap, 0.0]) / math.sqrt(2)
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        x1 = x0 + np.array([w0, 1.0 - w0])     # W_o = I; FFN off
        s = unit(x1) * np.array([1.0, 2.0])
        assert np.allclose(tr[j - 1], s, rtol=1e-12, atol=1e-12), f"sub-step {j}"
        hh = s                                 # W_back = I


def pin_layer_ffn(O):
    """Attention residual, then the gated FFN on rms(x) n2: with the mean-value attention of a
    zero query (W_o = I) and W_g = W_u = W_d = I, x2 = x1 + silu(b) b with b = rms(x1) n2."""
    cfg = micro_cfg()
    length = 2
    cache = cache_with(cfg, 8, [[[1.0, -1.0], [3.0, 1.0]]], [[[5.0, 5.0], [5.0, 5.0]]])
    lay = zero_layer(cfg)
    lay["wo"] = np.eye(2)
    lay["n1"] = np.array([3.0, 0.5])
    lay["n2"] = np.array([0.5, 2.0])
    lay["wg"] = lay["wu"] = lay["wd"] = np.eye(2)
    DW = drafter(cfg, [[1, 0, 0, 0], [0, 1, 0, 0]], [lay])
    h = np.array([2.0, 1.0])
    tr = []
    O.drafter_substep(DW, cfg, cache, h, 0, length, length, "full", 1, tr)
    x1 = unit(h) + np.array([2.0, 0.0])
    b = unit(x1) * lay["n2"]
    x2 = x1 + b / (1.0 + np.exp(-b)) * b
    assert np.allclose(tr[0], unit(x2), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# An independent drafter: explicit loops over elements, heads and keys; the input projection
# split into its hidden and token column blocks; rotary embedding as a complex rotation of
# (x_i + i x_{i+hd/2}); the clustered head by sorting clusters and scanning members.
# ---------------------------------------------------------------------------------------------

def _rms(v, w, eps):
    r = math.sqrt(sum(a * a for a in v) / len(v) + eps)
    return [a / r * wi for a, wi in zip(v, w)]


def _matvec(M, v):
    return [sum(M[r][c] * v[c] for c in range(len(v))) for r in range(len(M))]


def explicit_draft(DW, cfg, cache, hid, c0, length, K, head_mode, k_c):
    d, D, hd, Hq = cfg.d_model, cfg.d_dim, cfg.head_dim, cfg.n_q_heads
    G, half, eps = cfg.n_q_heads // cfg.n_kv_heads, cfg.head_dim // 2, cfg.rms_eps
    Kc, Vc = cache.K[cfg.n_layers - 1], cache.V[cfg.n_layers - 1]
    W_in = DW["w_in"].tolist()
    h, c, toks, states, hiddens = list(hid), int(c0), [], [], []
    for j in range(1, K + 1):
        uh = _rms(h, DW["norm_h"], eps)
        ue = _rms(DW["table"][c].tolist(), DW["norm_e"], eps)
        x = [sum(W_in[r][i] * uh[i] for i in range(d)) + sum(W_in[r][d + i] * ue[i] for i in range(D))
             for r in range(D)]
        t = length + j - 1
        for lw in DW["layers"]:
            a = _rms(x, lw["n1"], eps)
            q = _matvec(lw["wq"].tolist(), a)
            o = []
            for hh in range(Hq):
                qh = q[hh * hd:(hh + 1) * hd]
                rot = list(qh)
                for i in range(half):
                    z = complex(qh[i], qh[i + half]) * cmath.exp(1j * t * cfg.rope_theta ** (-2.0 * i / hd))
                    rot[i], rot[i + half] = z.real, z.imag
                g = hh // G
                sc = [sum(rot[e] * Kc[g, p, e] for e in range(hd)) / math.sqrt(hd) for p in range(length)]
                mx = max(sc)
                ex = [math.exp(v - mx) for v in sc]
                tot = sum(ex)
                o.extend(sum(ex[p] / tot * Vc[g, p, e] for p in range(length)) for e in range(hd))
            x = [xi + yi for xi, yi in zip(x, _matvec(lw["wo"].tolist(), o))]
            b = _rms(x, lw["n2"], eps)
            gt = _matvec(lw["wg"].tolist(), b)
            up = _matvec(lw["wu"].tolist(), b)
            hcat = [gv / (1.0 + math.exp(-gv)) * uv for gv, uv in zip(gt, up)]
            x = [xi + yi for xi, yi in zip(x, _matvec(lw["wd"].tolist(), hcat))]
        s = _rms(x, DW["norm_f"], eps)
        score = lambda tok: sum(DW["table"][tok][e] * s[e] for e in range(D))  # noqa: E731
        if head_mode == "full":
            cands = range(cfg.vocab)
        else:
            S = cfg.vocab // cfg.n_centroids
            zc = [sum(DW["centroids"][k][e] * s[e] for e in range(D)) for k in range(cfg.n_centroids)]
            chosen = sorted(range(cfg.n_centroids), key=lambda k: (-zc[k], k))[:k_c]
            cands = sorted(int(v) for k in chosen for v in DW["perm"][k * S:(k + 1) * S])
        best = None
        for tok in cands:  # ascending vocab id: the first maximum wins ties
            if best is None or score(tok) > score(best):
                best = tok
        toks.append(best)
        states.append(np.array(s))
        h = _matvec(DW["w_back"].tolist(), s)
        hiddens.append(np.array(h))
        c = best
    return toks, states, hiddens


RAND_CFG = ModelConfig(name="drafter-rand", n_layers=2, d_model=16, n_q_heads=4, n_kv_heads=2,
                       head_dim=8, ffn_dim=32, vocab=32, d_layers=2, d_dim=8, d_ffn=16,
                       n_centroids=4, dtype="f32", init="normal", rms_eps=1e-6)


def random_drafter(cfg, seed):
    rng = np.random.default_rng(seed)
    D, d, qd, F = cfg.d_dim, cfg.d_model, cfg.q_dim, cfg.d_ffn
    table = rng.normal(0, 0.5, (cfg.vocab, D))
    perm = rng.permutation(cfg.vocab)
    S = cfg.vocab // cfg.n_centroids
    DW = {"table": table, "perm": perm, "centroids": table[perm].reshape(cfg.n_centroids, S, D).mean(1),
          "norm_h": 1 + 0.3 * rng.uniform(-1, 1, d), "norm_e": 1 + 0.3 * rng.uniform(-1, 1, D),
          "w_in": rng.normal(0, 0.4, (D, d + D)), "norm_f": 1 + 0.3 * rng.uniform(-1, 1, D),
          "w_back": rng.normal(0, 0.6, (d, D)), "layers": []}
    for _ in range(cfg.d_layers):
        DW["layers"].append({"n1": 1 + 0.3 * rng.uniform(-1, 1, D), "wq": rng.normal(0, 0.5, (qd, D)),
                             "wo": rng.normal(0, 0.4, (D, qd)), "n2": 1 + 0.3 * rng.uniform(-1, 1, D),
                             "wg": rng.normal(0, 0.5, (F, D)), "wu": rng.normal(0, 0.5, (F, D)),
                             "wd": rng.normal(0, 0.4, (D, F))})
    length = 7
    cache = O.KVCache.empty(cfg, 16)
    for l in range(cfg.n_layers):
        cache.K[l][:, :length] = rng.normal(0, 1.0, (cfg.n_kv_heads, length, cfg.head_dim))
        cache.V[l][:, :length] = rng.normal(0, 1.0, (cfg.n_kv_heads, length, cfg.head_dim))
        cache.K[l][:, length:] = np.nan
        cache.V[l][:, length:] = np.nan
    hid = rng.normal(0, 1.0, d)
    return DW, cache, hid, length


def pin_explicit_agreement(O):
    """The oracle's drafter agrees with the explicit-loop drafter on random micro weights, for
    every head mode, to rounding: tokens exactly, head inputs and next hidden states within 1e-10."""
    cfg = RAND_CFG
    for seed in (1, 2, 3):
        DW, cache, hid, length = random_drafter(cfg, seed)
        for mode, k_c in (("full", 1), ("clustered", 1), ("clustered", 2), ("clustered", 4)):
            ref_t, ref_s, ref_h = explicit_draft(DW, cfg, cache, hid, 5, length, 3, mode, k_c)
            tr = []
            got = O.draft(DW, cfg, cache, hid, 5, length, 3, head_mode=mode, k_c=k_c, trace=tr)
            assert got == ref_t, (seed, mode, k_c)
            for j in range(3):
                assert np.allclose(tr[j], ref_s[j], rtol=1e-10, atol=1e-10)
            # the next hidden state of sub-step j is the input of sub-step j+1: check the last one
            _, hn = O.drafter_substep(DW, cfg, cache, ref_h[1], got[1], length + 2, length, mode, k_c)
            assert np.allclose(hn, ref_h[2], rtol=1e-10, atol=1e-10)


PINS = [pin_input_wiring, pin_source_layer_key_range_and_grouping, pin_rope_position,
        pin_layer_ffn, pin_explicit_agreement]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_drafter_pin(pin):
    pin(O)


# Each planted mistake: (name, text in the oracle's source, replacement).
MUTANTS = [
    ("concat order reversed",
     'u = np.concatenate([rmsnorm(h, DW["norm_h"], cfg.rms_eps), rmsnorm(e, DW["norm_e"], cfg.rms_eps)])',
     'u = np.concatenate([rmsnorm(e, DW["norm_e"], cfg.rms_eps), rmsnorm(h, DW["norm_h"], cfg.rms_eps)])'),
    ("rotary at len + j",
     "c, h = drafter_substep(DW, cfg, cache, h, c, length + j - 1, length, head_mode, k_c, trace)",
     "c, h = drafter_substep(DW, cfg, cache, h, c, length + j, length, head_mode, k_c, trace)"),
    ("source layer 0",
     "Ks = cache.K[cfg.src_layer][:, :length]\n    Vs = cache.V[cfg.src_layer][:, :length]",
     "Ks = cache.K[0][:, :length]\n    Vs = cache.V[0][:, :length]"),
    ("token norm weight dropped",
     'rmsnorm(e, DW["norm_e"], cfg.rms_eps)', 'rmsnorm(e, 1.0, cfg.rms_eps)'),
    ("hidden norm weight dropped",
     'rmsnorm(h, DW["norm_h"], cfg.rms_eps)', 'rmsnorm(h, 1.0, cfg.rms_eps)'),
    ("W_back applied to x",
     'return d, DW["w_back"] @ s', 'return d, DW["w_back"] @ x'),
    ("key range [0, len]",
     "Ks = cache.K[cfg.src_layer][:, :length]\n    Vs = cache.V[cfg.src_layer][:, :length]",
     "Ks = cache.K[cfg.src_layer][:, :length + 1]\n    Vs = cache.V[cfg.src_layer][:, :length + 1]"),
    ("first norm for the FFN",
     'b = rmsnorm(x, lw["n2"], cfg.rms_eps)', 'b = rmsnorm(x, lw["n1"], cfg.rms_eps)'),
    ("final norm weight dropped",
     's = rmsnorm(x, DW["norm_f"], cfg.rms_eps)', 's = rmsnorm(x, 1.0, cfg.rms_eps)'),
]


def mutant_module(old, new):
    src = open(os.path.join(ROOT, "oracle", "model.py")).read()
    assert src.count(old) >= 1, f"planted-mistake anchor not found in the oracle: {old!r}"
    name = "oracle_mutant"
    mod = types.ModuleType(name)
    sys.modules[name] = mod
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_drafter_mistake_fails_a_pin(name, old, new):
    M = mutant_module(old, new)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(M)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no drafter pin catches: {name}"
