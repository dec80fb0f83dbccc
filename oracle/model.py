"""Float64 numpy oracle: target decoder, plain greedy decoding, MTP drafter,
clustered head, acceptance, commit and the speculative loop.

Sources (the pages are five web pages on Gemma 4's MTP drafters):
  [digest]  "Accelerating Gemma 4: faster inference with multi-token prediction drafters"
  [note]    "Gemma 4 MTP Drafter" (Obsidian note)
  [blog]    "Gemma 4 inference 3x faster? The announcement, dissected"
  [pixel]   "Accelerating Gemini Nano on Pixel with frozen multi-token prediction"
  [guide]   "Gemma 4's MTP drafter explained: speculative decoding with llama.cpp"

Readings where the pages are silent (decoder details, drafter wiring, cluster
construction, tie-breaks) are the plainest ones the rest supports; each is
named at the function that takes it.

TEST INFRASTRUCTURE ONLY: not imported by the HIP path.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from workloads import ExpertStack, Q4Codes, inject_draw, inject_threshold

__all__ = [
    "as_f64", "q4_weights", "rmsnorm", "silu", "rope", "attention", "dense_ffn", "moe_ffn", "moe_route",
    "moe_route_margin",
    "KVCache", "decoder_layer_row", "target_row", "lm_head", "argmax_first", "top2_margin",
    "greedy_generate", "prefill", "verify", "accept", "commit", "token_scores",
    "centroid_scores", "head_full",
    "head_clustered", "drafter_substep", "draft", "inject", "spec_generate", "SpecStats",
    "tree_parents", "tree_path", "head_top", "draft_tree", "inject_tree", "verify_tree",
    "accept_tree", "commit_tree", "spec_generate_tree",
]


def q4_weights(codes: np.ndarray, steps: np.ndarray) -> np.ndarray:
    """Weights of a matrix stored in 4-bit blocks ([guide] "Step 1 -- repackaging the QAT
    drafter": the QAT weights keep every 32-weight block of a matrix on a 4-bit grid, which is
    Q4_0's own layout).  Reading of Q4_0: along each row, block j of 32 consecutive weights has
    one fp16 step d_j and 4-bit codes q in 0..15, weight = d_j * (q - 8).  codes [..., K],
    steps [..., K/32]; float64 result (exact: an fp16 value times a small integer)."""
    q = np.asarray(codes)
    d = np.asarray(steps, dtype=np.float16).astype(np.float64)
    K = q.shape[-1]
    assert K % 32 == 0 and d.shape == q.shape[:-1] + (K // 32,)
    blocks = q.reshape(*q.shape[:-1], K // 32, 32).astype(np.float64) - 8.0
    return (blocks * d[..., None]).reshape(q.shape)


class _F64Stack:
    """A lazily generated expert stack whose slices come out as float64 weights."""

    def __init__(self, stack):
        self.stack = stack

    def __len__(self):
        return len(self.stack)

    def __getitem__(self, e):
        return as_f64(self.stack[e])


def as_f64(tree):
    """Recursively convert the weights of a weight dict to float64 (integer arrays kept); 4-bit
    tensors become their weights (q4_weights)."""
    if isinstance(tree, dict):
        return {k: as_f64(v) for k, v in tree.items()}
    if isinstance(tree, list):
        return [as_f64(v) for v in tree]
    if isinstance(tree, Q4Codes):
        return q4_weights(tree.codes, tree.steps)
    if isinstance(tree, ExpertStack):
        return _F64Stack(tree)
    if isinstance(tree, np.ndarray) and tree.dtype.kind == "f":
        return tree.astype(np.float64)
    return tree


# ---------------------------------------------------------------------------
# Decoder building blocks.  The workloads specify an RMSNorm / RoPE / gated-FFN
# decoder; the pages presuppose a standard autoregressive decoder that reads
# all weights per forward pass ([guide] "Why is generating tokens one at a time
# slow?"; [note] "Why is it needed").  Reading: pre-norm, eps 1e-6 with the
# weight applied as x*w, SiLU gate, RoPE theta 1e4 with rotate-half pairs
# (i, i + hd/2), score scale 1/sqrt(hd), no biases or soft-caps.
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate pairs (i, i + hd/2) of each head vector by pos * theta^(-2i/hd).  x: [H][hd]."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one position.

    q: [Hq][hd]; K, V: [Hkv][n][hd] (the n visible keys).  Query head h reads KV
    head h // (Hq/Hkv).  Softmax of q.k/sqrt(hd) with the max subtracted.
    """
    Hq, hd = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.empty((Hq, hd), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    for h in range(Hq):
        g = h // G
        s = (K[g] @ q[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        p /= p.sum()
        out[h] = p @ V[g]
    return out


def dense_ffn(wg, wu, wd, b):
    """Gated FFN: Wd (silu(Wg b) * (Wu b))."""
    return wd @ (silu(wg @ b) * (wu @ b))


def moe_route(router: np.ndarray, b: np.ndarray, top_k: int):
    """Top-k experts by router logit (ties -> lower expert id) and softmax weights over them.

    Returned in ascending expert id, the order in which expert outputs are summed.
    """
    r = router @ b
    order = sorted(range(r.shape[0]), key=lambda e: (-r[e], e))[:top_k]
    sel = np.array(sorted(order), dtype=np.int64)
    z = r[sel] - r[sel].max()
    w = np.exp(z)
    w /= w.sum()
    return sel, w


def moe_route_margin(router: np.ndarray, b: np.ndarray, top_k: int) -> float:
    """Gap between the top_k-th largest router logit and the next one.  The expert choice is an
    integer decided from floating-point logits: where this gap is within the logits' rounding
    error, either choice is a correct result."""
    r = np.sort(router @ b)[::-1]
    return float(r[top_k - 1] - r[top_k]) if top_k < r.shape[0] else math.inf


def moe_ffn(lw: dict, cfg, b: np.ndarray, trace: list | None = None) -> np.ndarray:
    """Mixture-of-experts FFN: sum over the top-k experts (ascending id) of w_e * FFN_e(b), plus a
    shared gated FFN that every token uses.  The pages say only that the 26B MoE has a batch-1
    "routing challenge" ([digest] "Inside the MTP drafter"); routing details are a reading.
    `trace`, when given, receives the routing margin (moe_route_margin)."""
    if trace is not None:
        trace.append(moe_route_margin(lw["router"], b, cfg.top_k))
    sel, w = moe_route(lw["router"], b, cfg.top_k)
    y = np.zeros_like(b)
    for e, we in zip(sel, w):
        y = y + we * dense_ffn(lw["exp_wg"][e], lw["exp_wu"][e], lw["exp_wd"][e], b)
    return y + dense_ffn(lw["sh_wg"], lw["sh_wu"], lw["sh_wd"], b)


@dataclass
class KVCache:
    """Target KV cache of one sequence: K[l], V[l] arrays [Hkv][cap][hd] (float64).

    Entries at positions >= the committed length are dead: a rollback is only a
    length reset ([pixel] "The 'late exit' strategy": return to the first mismatch).
    """

    K: list
    V: list

    @classmethod
    def empty(cls, cfg, cap: int) -> "KVCache":
        shp = (cfg.n_kv_heads, cap, cfg.head_dim)
        return cls([np.zeros(shp) for _ in range(cfg.n_layers)],
                   [np.zeros(shp) for _ in range(cfg.n_layers)])

    @classmethod
    def from_synthetic(cls, cfg, k: np.ndarray, v: np.ndarray, cap: int) -> "KVCache":
        """Cache whose first k.shape[2] positions hold the given [L][Hkv][n][hd] keys / values."""
        c = cls.empty(cfg, cap)
        n = k.shape[2]
        for l in range(cfg.n_layers):
            c.K[l][:, :n] = k[l]
            c.V[l][:, :n] = v[l]
        return c

    def copy(self) -> "KVCache":
        return KVCache([a.copy() for a in self.K], [a.copy() for a in self.V])


def decoder_layer_row(lw: dict, cfg, Kl: np.ndarray, Vl: np.ndarray, x: np.ndarray,
                      pos: int, trace: list | None = None) -> np.ndarray:
    """One decoder layer for one token at position pos.  Writes k, v at pos, attends keys [0, pos].
    `trace` (mixture of experts only) receives the layer's routing margin."""
    hd = cfg.head_dim
    a = rmsnorm(x, lw["attn_norm"], cfg.rms_eps)
    q = (lw["wq"] @ a).reshape(cfg.n_q_heads, hd)
    k = (lw["wk"] @ a).reshape(cfg.n_kv_heads, hd)
    v = (lw["wv"] @ a).reshape(cfg.n_kv_heads, hd)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    Kl[:, pos] = k
    Vl[:, pos] = v
    o = attention(q, Kl[:, : pos + 1], Vl[:, : pos + 1])
    x = x + lw["wo"] @ o.reshape(-1)
    b = rmsnorm(x, lw["ffn_norm"], cfg.rms_eps)
    if cfg.is_moe:
        return x + moe_ffn(lw, cfg, b, trace)
    return x + dense_ffn(lw["wg"], lw["wu"], lw["wd"], b)


def lm_head(W: dict, cfg, hidden: np.ndarray) -> np.ndarray:
    """Tied output layer: logits = E . rmsnorm(hidden), for one hidden row [d] or a stack of
    rows [n][d] (then [n][V]).  Reading: the LM head is tied to the embedding (the 31B workload's
    ~30.5B parameter count only matches a tied head)."""
    return rmsnorm(hidden, W["final_norm"], cfg.rms_eps) @ W["embed"].T


def target_row(W: dict, cfg, cache: KVCache, tok: int, pos: int):
    """Target forward for one token at position pos (O2): returns (logits [V], hidden [d]).

    hidden is the residual stream after the last layer, before the final norm.
    """
    x = W["embed"][tok].copy()
    for l, lw in enumerate(W["layers"]):
        x = decoder_layer_row(lw, cfg, cache.K[l], cache.V[l], x, pos)
    return lm_head(W, cfg, x), x


def argmax_first(v: np.ndarray) -> int:
    """Index of the maximum; the lowest index wins ties.  NaN raises."""
    if np.isnan(v).any():
        raise FloatingPointError("NaN in logits")
    return int(np.argmax(v))


def top2_margin(v: np.ndarray) -> float:
    """Gap between the largest and the second-largest entry."""
    t = np.partition(v, -2)[-2:]
    return float(t[1] - t[0])


def prefill(W: dict, cfg, cache: KVCache, prompt) -> tuple[int, np.ndarray, int]:
    """Feed the prompt row by row ([note] "How it works": the target processes the prompt
    first).  Returns (first generated token, hidden of the last prompt row, length)."""
    logits = hidden = None
    for pos, tok in enumerate(prompt):
        logits, hidden = target_row(W, cfg, cache, int(tok), pos)
    return argmax_first(logits), hidden, len(prompt)


def greedy_generate(W: dict, cfg, cache: KVCache, t0: int, length: int, n: int,
                    record_margins: bool = False):
    """Plain greedy decoding (O3): one token per full forward pass ([guide] "Why is generating
    tokens one at a time slow?").  Starts with t0 at position `length`; returns the n tokens
    t0, g1, ..., g_{n-1} (t0 included) and optionally each step's top-2 logit margin."""
    toks = [int(t0)]
    margins = []
    pos = length
    while len(toks) < n:
        logits, _ = target_row(W, cfg, cache, toks[-1], pos)
        margins.append(top2_margin(logits))
        toks.append(argmax_first(logits))
        pos += 1
    return (toks, margins) if record_margins else toks


def verify(W: dict, cfg, cache: KVCache, length: int, T) -> tuple[list, list, list]:
    """Verify pass (O4): the target scores the current token and the K drafts, all in one pass
    ([guide] "How does speculative decoding work?").  Row i is token T[i] at position length+i
    and sees keys [0, length+i].  Written as the decode step applied row by row, so every row
    is exactly the row plain greedy decoding would compute.  Returns (G, H, logits)."""
    G, H, Ls = [], [], []
    for i, tok in enumerate(T):
        logits, hidden = target_row(W, cfg, cache, int(tok), length + i)
        G.append(argmax_first(logits))
        H.append(hidden)
        Ls.append(logits)
    return G, H, Ls


def accept(T, G) -> tuple[int, list, int]:
    """Acceptance (O5): drafts T[1..K] are kept up to the first one the target disagrees with;
    the rest are dropped and the target's own token at that point is appended
    ([guide] "How does speculative decoding work?"; [digest] "How MTP works": one extra token).

    m = largest j <= K with T[1..j] == G[0..j-1].  Returns (m, emitted = T[1..m] + [G[m]], next).
    """
    K = len(T) - 1
    m = 0
    while m < K and int(T[m + 1]) == int(G[m]):
        m += 1
    out = [int(t) for t in T[1 : m + 1]] + [int(G[m])]
    return m, out, int(G[m])


def commit(cache: KVCache | None, length: int, n_rows: int, m: int, H, poison: bool = False):
    """Commit / rollback (O6): the committed length grows by m+1 and the drafter's hidden input
    becomes H[m] ([pixel] "The 'late exit' strategy": roll back to the first mismatch).  With
    poison=True the dead slots [length+m+1, length+n_rows) are overwritten with NaN, which any
    later read of them would propagate."""
    new_len = length + m + 1
    if poison and cache is not None:
        for l in range(len(cache.K)):
            cache.K[l][:, new_len : length + n_rows] = np.nan
            cache.V[l][:, new_len : length + n_rows] = np.nan
    return new_len, H[m]


# ---------------------------------------------------------------------------
# Drafter.  The pages: a light 4-layer head, width 256, that reads the target's
# last hidden state ("backbone_hidden_size") and activations, cross-attends to the
# target's KV cache and keeps no cache of its own, and predicts future tokens
# autoregressively ([guide] "What is different about Gemma 4's drafter?";
# [pixel] "The 'late exit' strategy" and "Zero-copy architecture").  Its output
# layer has a clustered shortcut (num_centroids 2048) that can be dropped for
# full-vocabulary scoring (same [guide] section; [digest] "Inside the MTP drafter").
# ---------------------------------------------------------------------------

def token_scores(table: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Score of every token the table lists: table[t] . s."""
    return table @ s


def centroid_scores(centroids: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Score of every cluster: centroids[c] . s."""
    return centroids @ s


def head_full(table: np.ndarray, s: np.ndarray) -> int:
    """Full-vocabulary scoring: argmax over t of table[t] . s (lowest vocab id on ties)."""
    return argmax_first(token_scores(table, s))


def head_clustered(table: np.ndarray, centroids: np.ndarray, perm: np.ndarray, s: np.ndarray,
                   k_c: int) -> int:
    """Clustered output layer.  Score the centroids, keep the k_c best clusters (ties -> lower
    cluster id), then take the argmax of table[t] . s over the member tokens of those clusters
    (ties -> lower vocab id).  Cluster c's members are perm[c*S:(c+1)*S].  Reading: clusters of
    equal size from a seeded permutation, centroid = member mean."""
    Nc = centroids.shape[0]
    S = table.shape[0] // Nc
    z = centroid_scores(centroids, s)
    sel = sorted(range(Nc), key=lambda c: (-z[c], c))[:k_c]
    cand = np.sort(np.concatenate([perm[c * S:(c + 1) * S] for c in sel]))
    scores = token_scores(table[cand], s)
    if np.isnan(scores).any():
        raise FloatingPointError("NaN in drafter scores")
    best = int(np.argmax(scores))  # cand is sorted, so the first max is the lowest vocab id
    return int(cand[best])


def drafter_substep(DW: dict, cfg, cache: KVCache, h: np.ndarray, c_prev: int, qpos: int,
                    length: int, head_mode: str = "clustered", k_c: int = 1, trace=None):
    """One drafter sub-step: returns (draft token, next hidden input).

    Readings: input x = W_in [rms(h)*n_h ; rms(table[c_prev])*n_e]; each drafter layer is
    RMSNorm -> q projection -> RoPE at qpos -> cross-attention over the target's layer-l* KV,
    keys [0, length), with the target's GQA grouping -> O projection + residual -> RMSNorm ->
    gated FFN + residual.  s = rms(x)*n_f scores the head; the next hidden is W_back s.
    """
    e = DW["table"][c_prev]
    u = np.concatenate([rmsnorm(h, DW["norm_h"], cfg.rms_eps), rmsnorm(e, DW["norm_e"], cfg.rms_eps)])
    x = DW["w_in"] @ u
    Ks = cache.K[cfg.src_layer][:, :length]
    Vs = cache.V[cfg.src_layer][:, :length]
    for lw in DW["layers"]:
        a = rmsnorm(x, lw["n1"], cfg.rms_eps)
        q = (lw["wq"] @ a).reshape(cfg.n_q_heads, cfg.head_dim)
        q = rope(q, qpos, cfg.rope_theta)
        o = attention(q, Ks, Vs)
        x = x + lw["wo"] @ o.reshape(-1)
        b = rmsnorm(x, lw["n2"], cfg.rms_eps)
        x = x + dense_ffn(lw["wg"], lw["wu"], lw["wd"], b)
    s = rmsnorm(x, DW["norm_f"], cfg.rms_eps)
    if trace is not None:
        trace.append(s)
    if head_mode == "full":
        d = head_full(DW["table"], s)
    else:
        d = head_clustered(DW["table"], DW["centroids"], DW["perm"], s, k_c)
    return d, DW["w_back"] @ s


def draft(DW: dict, cfg, cache: KVCache, hid: np.ndarray, c0: int, length: int, K: int,
          head_mode: str = "clustered", k_c: int = 1, trace=None) -> list:
    """Draft K tokens (O7).  Sub-step j (1..K) reads the token c_{j-1} at position length+j-1
    (c_0 is the current token, not yet in the cache) and proposes the token at length+j."""
    h = hid
    c = int(c0)
    out = []
    for j in range(1, K + 1):
        c, h = drafter_substep(DW, cfg, cache, h, c, length + j - 1, length, head_mode, k_c, trace)
        out.append(c)
    return out


def inject(drafts, greedy_seq, length: int, p: float, seed: int, b: int = 0,
           forced_wrong: bool = False, vocab: int | None = None) -> list:
    """Workload injection (O9), applied after drafting: draft j (proposing absolute position
    length+j) becomes greedy_seq[length+j] when its 53-bit draw is below floor(p*2^53).  The
    forced-wrong variant uses (greedy_seq[length+j] + 1) mod V for every slot instead."""
    out = list(drafts)
    if forced_wrong:
        return [(int(greedy_seq[length + j]) + 1) % vocab for j in range(1, len(out) + 1)]
    thr = inject_threshold(p)
    for j in range(1, len(out) + 1):
        if inject_draw(seed, b, length + j, j) < thr:
            out[j - 1] = int(greedy_seq[length + j])
    return out


@dataclass
class SpecStats:
    steps: int = 0
    proposed: int = 0
    accepted: int = 0
    emitted_per_step: list = field(default_factory=list)

    @property
    def tokens_per_pass(self) -> float:
        return sum(self.emitted_per_step) / max(self.steps, 1)


def spec_generate(W: dict, DW: dict, cfg, cache: KVCache, t0: int, hid: np.ndarray, length: int,
                  n: int, K: int, greedy_seq=None, p: float = 0.0, seed: int = 0,
                  head_mode: str = "clustered", k_c: int = 1, forced_wrong: bool = False,
                  poison: bool = False, b: int = 0):
    """Speculative loop (O10): draft -> (inject) -> verify -> accept -> commit until n tokens.

    Starts like greedy_generate (t0 at position `length` is the first token) and returns
    exactly n tokens; the last step is truncated.  Without EOS.
    """
    toks = [int(t0)]
    st = SpecStats()
    cur = int(t0)
    while len(toks) < n:
        d = draft(DW, cfg, cache, hid, cur, length, K, head_mode, k_c)
        if greedy_seq is not None:
            d = inject(d, greedy_seq, length, p, seed, b, forced_wrong, cfg.vocab)
        T = [cur] + d
        G, H, _ = verify(W, cfg, cache, length, T)
        m, out, cur = accept(T, G)
        length, hid = commit(cache, length, K + 1, m, H, poison=poison)
        toks.extend(out)
        st.steps += 1
        st.proposed += K
        st.accepted += m
        st.emitted_per_step.append(m + 1)
    return toks[:n], st


# ---------------------------------------------------------------------------
# Token trees.  Standard speculative decoding bets on one future path; the Pixel
# page's "Future directions" describe letting the drafter explore branching
# possibilities in parallel so a long sequence is accepted more often when the
# context is uncertain.  Reading: the first drafter sub-step's `width` best
# tokens start `width` branches, each continued greedily for `depth` tokens;
# the target scores every node as the next token after its root-to-node path;
# acceptance follows, from the root, the child equal to the target's token.
# ---------------------------------------------------------------------------

def tree_parents(width: int, depth: int) -> list:
    """Parent of every node of the width x depth branch tree, in node order: node 0 is the
    root; node 1 + width*(j-1) + k is the j-th token of branch k."""
    par = [-1]
    for j in range(1, depth + 1):
        for k in range(width):
            par.append(0 if j == 1 else 1 + width * (j - 2) + k)
    return par


def tree_path(parent, i: int) -> list:
    """Nodes from the root to node i (both included)."""
    path = [i]
    while parent[path[-1]] >= 0:
        path.append(parent[path[-1]])
    return path[::-1]


def head_top(DW: dict, s: np.ndarray, width: int, head_mode: str = "clustered", k_c: int = 1) -> list:
    """The `width` best tokens among those the head scores (the members of the k_c best clusters,
    or every token), by score and then lower vocabulary id."""
    table = DW["table"]
    if head_mode == "full":
        cand = np.arange(table.shape[0])
    else:
        Nc = DW["centroids"].shape[0]
        S = table.shape[0] // Nc
        z = centroid_scores(DW["centroids"], s)
        sel = sorted(range(Nc), key=lambda c: (-z[c], c))[:k_c]
        cand = np.concatenate([DW["perm"][c * S:(c + 1) * S] for c in sel])
    sc = token_scores(table[cand], s)
    if np.isnan(sc).any():
        raise FloatingPointError("NaN in drafter scores")
    order = sorted(range(len(cand)), key=lambda i: (-sc[i], int(cand[i])))
    return [int(cand[i]) for i in order[:width]]


def draft_tree(DW: dict, cfg, cache: KVCache, hid: np.ndarray, c0: int, length: int, width: int,
               depth: int, head_mode: str = "clustered", k_c: int = 1) -> list:
    """Tokens of every node of a width x depth tree draft, in node order (node 0 = c0)."""
    st = []
    _, h1 = drafter_substep(DW, cfg, cache, hid, c0, length, length, head_mode, k_c, st)
    firsts = head_top(DW, st[0], width, head_mode, k_c)
    toks = [int(c0)] + firsts
    branches = [[t] for t in firsts]
    hs = [h1] * width
    for j in range(2, depth + 1):
        for k in range(width):
            d, hs[k] = drafter_substep(DW, cfg, cache, hs[k], branches[k][-1], length + j - 1,
                                       length, head_mode, k_c)
            branches[k].append(d)
        toks.extend(branches[k][-1] for k in range(width))
    return toks


def inject_tree(tokens, parent, greedy_seq, length: int, p: float, seed: int, b: int = 0) -> list:
    """Workload injection for a tree: the node at depth j in slot s = node - 1 becomes
    greedy_seq[length + j] when its draw (the linear one with slot s + 1 for j) is below p."""
    out = list(tokens)
    thr = inject_threshold(p)
    depth = [0] * len(parent)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
        if inject_draw(seed, b, length + depth[i], i) < thr:
            out[i] = int(greedy_seq[length + depth[i]])
    return out


def verify_tree(W: dict, cfg, cache: KVCache, length: int, tokens, parent):
    """Every node of a tree scored by the target as plain decoding of its root-to-node path would
    score it (the path's tokens at positions length, length + 1, ...).  Returns (G, H, logits)
    per node; the cache is not changed."""
    G, H, Ls = [], [], []
    for i in range(len(tokens)):
        c = cache.copy()
        logits = hidden = None
        for j, node in enumerate(tree_path(parent, i)):
            logits, hidden = target_row(W, cfg, c, int(tokens[node]), length + j)
        G.append(argmax_first(logits))
        H.append(hidden)
        Ls.append(logits)
    return G, H, Ls


def accept_tree(tokens, parent, G):
    """The longest root path on which every node's token is the target's choice at its parent
    (the tree's longest agreeing draft); among equally long paths the one with the lower node
    index at the first place they differ.  Written as a search over every node's root path.
    Returns (m, emitted = the path's tokens + [G at its last node], next, path nodes)."""
    best = []
    for i in range(len(tokens)):
        path = tree_path(parent, i)
        if all(int(tokens[path[j]]) == int(G[path[j - 1]]) for j in range(1, len(path))):
            cand = path[1:]
            if len(cand) > len(best) or (len(cand) == len(best) and cand < best):
                best = cand
    end = best[-1] if best else 0
    out = [int(tokens[n]) for n in best] + [int(G[end])]
    return len(best), out, int(G[end]), best


def commit_tree(W: dict, cfg, cache: KVCache, length: int, tokens, nodes, H):
    """The committed state after accepting a tree path: the root's and the path's keys and values
    at positions length .. length + m (what plain decoding of those tokens writes), the length
    grown by m + 1 and the hidden of the path's last node."""
    for j, node in enumerate([0] + list(nodes)):
        target_row(W, cfg, cache, int(tokens[node]), length + j)
    return length + len(nodes) + 1, H[nodes[-1] if nodes else 0]


def spec_generate_tree(W: dict, DW: dict, cfg, cache: KVCache, t0: int, hid: np.ndarray,
                       length: int, n: int, width: int, depth: int, greedy_seq=None, p: float = 0.0,
                       seed: int = 0, head_mode: str = "clustered", k_c: int = 1, b: int = 0):
    """The speculative loop with tree drafts: draft_tree -> (inject) -> verify_tree -> accept_tree
    -> commit, until n tokens (t0 first; the last step truncated)."""
    parent = tree_parents(width, depth)
    toks, cur, st = [int(t0)], int(t0), SpecStats()
    while len(toks) < n:
        T = draft_tree(DW, cfg, cache, hid, cur, length, width, depth, head_mode, k_c)
        if greedy_seq is not None:
            T = inject_tree(T, parent, greedy_seq, length, p, seed, b)
        G, H, _ = verify_tree(W, cfg, cache, length, T, parent)
        m, out, cur, nodes = accept_tree(T, parent, G)
        length, hid = commit_tree(W, cfg, cache, length, T, nodes, H)
        toks.extend(out)
        st.steps += 1
        st.proposed += depth
        st.accepted += m
        st.emitted_per_step.append(m + 1)
    return toks[:n], st
