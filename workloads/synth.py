"""Seeded synthetic input generators (host side, numpy).

Two generators are used:

* ``normal``: numpy ``default_rng([seed, tensor_id]).normal(0, std)`` in fp32,
  one independent stream per tensor (the tiny configuration's "fp32 N(0, 0.02)
  seeded weights").
* ``hash``: a counter-based generator built on SplitMix64 (Steele, Lea and Flood,
  "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014; the 64-bit
  finaliser is Stafford's "Mix13").  Element ``i`` of a stream with key ``k`` is
  the ``(i+1)``-th SplitMix64 output of state ``k``:
  ``mix64(k + (i+1) * 0x9E3779B97F4A7C15)``.  A uniform value on
  ``[-std*sqrt(3), +std*sqrt(3)]`` is formed from the top 24 bits as the odd
  integer ``2*u24 - (2^24 - 1)`` times the fp32 constant
  ``float32(std*sqrt(3) / 2^24)``; the one fp32 multiply rounds to nearest-even
  on every IEEE machine, and bf16 tensors then round that fp32 value to bf16
  nearest-even.  The HIP fill in ``workloads/csrc/synth_fill.hip`` implements the
  same definition, so device-generated tensors are bit-identical to these.

Weights in the 4-bit block format (``weight_format == "q4"``) are drawn as raw
codes and steps, not values: code ``i`` of a tensor is the top 4 bits of element
``i`` of its hash stream; the fp16 step of (row, 32-column block) ``j`` comes from
the stream of tensor id + 2^19, as
``float16(float32(u23 + 2^23) * float32(2*s / (3 * 2^23)))`` with ``u23`` the top 23
bits and ``s = std / sqrt(21.5)`` (21.5 = mean of (code - 8)^2 over uniform codes):
steps uniform on [2s/3, 4s/3).  The generators return them as ``Q4Codes``; turning
codes into weights is left to the consumers.

Draft injection (the workload's "replace drafts with the target's greedy token
with probability p") draws ``U = hash >> 11`` (53 bits) per (sequence, absolute
position, draft slot) and replaces iff ``U < floor(p * 2^53)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "GOLDEN", "mix64", "stream_key", "hash_u64", "hash_uniform_f32", "bf16_round",
    "bf16_bits", "bf16_from_bits", "TID", "tensor_id", "gen_tensor", "gen_rows",
    "norm_weight", "target_weights", "target_layer_weights", "drafter_weights",
    "cluster_perm", "centroids_from_table", "drafter_centroids", "kv_init", "kv_rows", "state_init",
    "prompt_tokens", "inject_threshold", "inject_draw", "inject_key", "hash_scale",
    "hash_u64_at", "inject_table", "ExpertStack", "Q4Codes", "gen_q4_rows", "q4_step_scale",
    "Q4_STEP_TID",
]

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_G = np.uint64(GOLDEN)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    """Key of stream ``tid`` under ``seed``: first SplitMix64 output of state seed*2^32+tid."""
    return _mix64_int(((seed << 32) + tid + GOLDEN) & MASK64)


def hash_u64(key: int, start: int, n: int) -> np.ndarray:
    """Elements ``start .. start+n-1`` of the counter stream with key ``key``."""
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + idx * _G)


def hash_u64_at(key: int, idx: np.ndarray) -> np.ndarray:
    """Elements at arbitrary indices of the counter stream with key ``key``."""
    i = np.asarray(idx, dtype=np.uint64) + np.uint64(1)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + i * _G)


def hash_scale(std: float) -> np.float32:
    return np.float32(std * math.sqrt(3.0) / float(1 << 24))


def hash_uniform_f32(key: int, start: int, n: int, std: float) -> np.ndarray:
    z = hash_u64(key, start, n)
    u24 = (z >> np.uint64(40)).astype(np.int64)
    odd = (2 * u24 - ((1 << 24) - 1)).astype(np.float32)
    return odd * hash_scale(std)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even); returns the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    with np.errstate(over="ignore"):
        return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_from_bits(bf16_bits(x))


# Stream ids.  tensor_id = TID[name] * 2^20 + layer.
TID = {
    "embed": 1, "final_norm": 2,
    "attn_norm": 10, "wq": 11, "wk": 12, "wv": 13, "wo": 14, "ffn_norm": 15,
    "wg": 16, "wu": 17, "wd": 18,
    "router": 19, "exp_wg": 20, "exp_wu": 21, "exp_wd": 22,
    "sh_wg": 23, "sh_wu": 24, "sh_wd": 25,
    "table": 40, "norm_h": 41, "norm_e": 42, "w_in": 43,
    "d_n1": 44, "d_wq": 45, "d_wo": 46, "d_n2": 47, "d_wg": 48, "d_wu": 49, "d_wd": 50,
    "d_nf": 51, "w_back": 52, "centroids": 53,
    "kv_k": 60, "kv_v": 61, "hid": 62, "tok": 63, "inject": 64,
}


def tensor_id(name: str, layer: int = 0) -> int:
    return TID[name] * (1 << 20) + layer


Q4_STEP_TID = 1 << 19  # the step stream of a 4-bit tensor: its tensor id + 2^19


@dataclass
class Q4Codes:
    """A weight tensor in the 4-bit block format as drawn: codes [..., K] (uint8, 0..15) and one
    fp16 step per 32 consecutive codes of a row, steps [..., K // 32] (float16)."""
    codes: np.ndarray
    steps: np.ndarray

    @property
    def shape(self):
        return self.codes.shape

    def __getitem__(self, idx) -> "Q4Codes":
        """Rows (leading-axis index or slice) of the tensor."""
        return Q4Codes(self.codes[idx], self.steps[idx])


def q4_step_scale(std: float) -> np.float32:
    return np.float32(2.0 * (std / math.sqrt(21.5)) / (3.0 * float(1 << 23)))


def gen_q4_rows(cfg, name: str, layer: int, n_cols: int, row_start: int, n_rows: int,
                std: float | None = None) -> Q4Codes:
    """Rows ``row_start .. row_start+n_rows-1`` of a 4-bit [*, n_cols] tensor (codes, steps)."""
    assert cfg.init == "hash" and n_cols % 32 == 0
    std = cfg.weight_std if std is None else std
    tid = tensor_id(name, layer)
    z = hash_u64(stream_key(cfg.seed, tid), row_start * n_cols, n_rows * n_cols)
    codes = (z >> np.uint64(60)).astype(np.uint8).reshape(n_rows, n_cols)
    nb = n_cols // 32
    zd = hash_u64(stream_key(cfg.seed, tid + Q4_STEP_TID), row_start * nb, n_rows * nb)
    u23 = (zd >> np.uint64(41)).astype(np.int64) + (1 << 23)
    steps = (u23.astype(np.float32) * q4_step_scale(std)).astype(np.float16).reshape(n_rows, nb)
    return Q4Codes(codes, steps)


def gen_rows(cfg, name: str, layer: int, n_cols: int, row_start: int, n_rows: int,
             std: float | None = None):
    """Rows ``row_start .. row_start+n_rows-1`` of a hash-initialised [*, n_cols] tensor (fp32
    values; ``Q4Codes`` for 4-bit weights)."""
    assert cfg.init == "hash"
    if cfg.weight_format == "q4":
        return gen_q4_rows(cfg, name, layer, n_cols, row_start, n_rows, std)
    std = cfg.weight_std if std is None else std
    key = stream_key(cfg.seed, tensor_id(name, layer))
    v = hash_uniform_f32(key, row_start * n_cols, n_rows * n_cols, std)
    if cfg.dtype == "bf16":
        v = bf16_round(v)
    return v.reshape(n_rows, n_cols)


def gen_tensor(cfg, name: str, layer: int, shape, std: float | None = None):
    """A weight tensor in logical row-major order, as fp32 values (bf16-representable for bf16);
    ``Q4Codes`` of that shape for 4-bit weights."""
    if cfg.weight_format == "q4":
        q = gen_q4_rows(cfg, name, layer, shape[-1], 0, int(np.prod(shape[:-1])), std)
        return Q4Codes(q.codes.reshape(shape), q.steps.reshape(*shape[:-1], shape[-1] // 32))
    std = cfg.weight_std if std is None else std
    n = int(np.prod(shape))
    if cfg.init == "normal":
        rng = np.random.default_rng([cfg.seed, tensor_id(name, layer)])
        v = rng.normal(0.0, std, size=n).astype(np.float32)
    else:
        key = stream_key(cfg.seed, tensor_id(name, layer))
        v = hash_uniform_f32(key, 0, n, std)
    if cfg.dtype == "bf16":
        v = bf16_round(v)
    return v.reshape(shape)


class ExpertStack:
    """A stacked [E][rows][cols] expert weight whose slices are generated on first use: with the
    hash generator each slice is its own range of the tensor's counter stream (identical to the
    slice of the whole tensor); with the normal generator the whole tensor is drawn once.
    Indexing by expert id returns that expert's [rows][cols] fp32 array (``Q4Codes`` for 4-bit
    weights)."""

    def __init__(self, cfg, name: str, layer: int, shape):
        self.cfg, self.name, self.layer, self.shape = cfg, name, layer, tuple(shape)
        self._full = None
        self._cache = {}

    def __len__(self) -> int:
        return self.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if not 0 <= e < self.shape[0]:
            raise IndexError(e)
        if self.cfg.init != "hash":
            if self._full is None:
                self._full = gen_tensor(self.cfg, self.name, self.layer, self.shape)
            return self._full[e]
        if e not in self._cache:
            _, r, c = self.shape
            self._cache[e] = gen_rows(self.cfg, self.name, self.layer, c, e * r, r)
        return self._cache[e]


def norm_weight(cfg, name: str, layer: int, n: int) -> np.ndarray:
    """RMSNorm weight: exactly 1, or 1 + jitter*U(-1, 1) when the workload asks for jitter."""
    if cfg.norm_jitter == 0.0:
        return np.ones(n, dtype=np.float32)
    key = stream_key(cfg.seed, tensor_id(name, layer))
    u = hash_uniform_f32(key, 0, n, 1.0 / math.sqrt(3.0))
    return (np.float32(1.0) + np.float32(cfg.norm_jitter) * u).astype(np.float32)


def target_layer_weights(cfg, l: int) -> dict:
    d, F = cfg.d_model, cfg.ffn_dim
    w = {
        "attn_norm": norm_weight(cfg, "attn_norm", l, d),
        "wq": gen_tensor(cfg, "wq", l, (cfg.q_dim, d)),
        "wk": gen_tensor(cfg, "wk", l, (cfg.kv_dim, d)),
        "wv": gen_tensor(cfg, "wv", l, (cfg.kv_dim, d)),
        "wo": gen_tensor(cfg, "wo", l, (d, cfg.q_dim)),
        "ffn_norm": norm_weight(cfg, "ffn_norm", l, d),
    }
    if cfg.is_moe:
        E, Fe, Fs = cfg.n_experts, cfg.expert_ffn, cfg.shared_ffn
        w["router"] = gen_tensor(cfg, "router", l, (E, d))
        w["exp_wg"] = ExpertStack(cfg, "exp_wg", l, (E, Fe, d))
        w["exp_wu"] = ExpertStack(cfg, "exp_wu", l, (E, Fe, d))
        w["exp_wd"] = ExpertStack(cfg, "exp_wd", l, (E, d, Fe))
        w["sh_wg"] = gen_tensor(cfg, "sh_wg", l, (Fs, d))
        w["sh_wu"] = gen_tensor(cfg, "sh_wu", l, (Fs, d))
        w["sh_wd"] = gen_tensor(cfg, "sh_wd", l, (d, Fs))
    else:
        w["wg"] = gen_tensor(cfg, "wg", l, (F, d))
        w["wu"] = gen_tensor(cfg, "wu", l, (F, d))
        w["wd"] = gen_tensor(cfg, "wd", l, (d, F))
    return w


def target_weights(cfg, with_embed: bool = True) -> dict:
    """All target weights in logical layout: embed [V][d] (tied LM head), final_norm [d], layers."""
    w = {
        "final_norm": norm_weight(cfg, "final_norm", 0, cfg.d_model),
        "layers": [target_layer_weights(cfg, l) for l in range(cfg.n_layers)],
    }
    if with_embed:
        w["embed"] = gen_tensor(cfg, "embed", 0, (cfg.vocab, cfg.d_model))
    return w


def cluster_perm(cfg) -> np.ndarray:
    """Seeded permutation of the vocabulary; cluster c holds perm[c*S:(c+1)*S], S = V / Nc."""
    return np.random.default_rng(cfg.perm_seed).permutation(cfg.vocab).astype(np.int64)


def centroids_from_table(cfg, table: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Centroid c = mean of its members' table rows, rounded to the storage dtype."""
    S = cfg.cluster_size
    members = table[perm].reshape(cfg.n_centroids, S, cfg.d_dim).astype(np.float64)
    c = members.mean(axis=1).astype(np.float32)
    return bf16_round(c) if cfg.dtype == "bf16" else c


def drafter_centroids(cfg, table, perm):
    """The clustered head's centroids: member means of the table for dense weights; for 4-bit
    weights a drawn 4-bit tensor of their own (stream "centroids")."""
    if cfg.weight_format == "q4":
        return gen_tensor(cfg, "centroids", 0, (cfg.n_centroids, cfg.d_dim))
    return centroids_from_table(cfg, table, perm)


def drafter_weights(cfg) -> dict:
    D, d, Fd = cfg.d_dim, cfg.d_model, cfg.d_ffn
    table = gen_tensor(cfg, "table", 0, (cfg.vocab, D))
    perm = cluster_perm(cfg)
    w = {
        "table": table,
        "perm": perm,
        "centroids": drafter_centroids(cfg, table, perm),
        "norm_h": norm_weight(cfg, "norm_h", 0, d),
        "norm_e": norm_weight(cfg, "norm_e", 0, D),
        "w_in": gen_tensor(cfg, "w_in", 0, (D, d + D)),
        "layers": [],
        "norm_f": norm_weight(cfg, "d_nf", 0, D),
        "w_back": gen_tensor(cfg, "w_back", 0, (d, D)),
    }
    for l in range(cfg.d_layers):
        w["layers"].append({
            "n1": norm_weight(cfg, "d_n1", l, D),
            "wq": gen_tensor(cfg, "d_wq", l, (cfg.q_dim, D)),
            "wo": gen_tensor(cfg, "d_wo", l, (D, cfg.q_dim)),
            "n2": norm_weight(cfg, "d_n2", l, D),
            "wg": gen_tensor(cfg, "d_wg", l, (Fd, D)),
            "wu": gen_tensor(cfg, "d_wu", l, (Fd, D)),
            "wd": gen_tensor(cfg, "d_wd", l, (D, Fd)),
        })
    return w


def kv_rows(cfg, which: str, layer: int, b: int, g: int, pos0: int, n: int) -> np.ndarray:
    """Synthetic committed KV (std 1, storage dtype) for positions pos0..pos0+n-1 of one head.

    Element (l, b, g, pos, c) has logical index (((l*B + b)*Hkv + g)*ctx + pos)*hd + c.
    """
    hd, ctx = cfg.head_dim, cfg.ctx
    key = stream_key(cfg.kv_seed, tensor_id("kv_k" if which == "k" else "kv_v", 0))
    base = (((layer * cfg.batch + b) * cfg.n_kv_heads + g) * ctx + pos0) * hd
    v = hash_uniform_f32(key, base, n * hd, 1.0)
    if cfg.dtype == "bf16":
        v = bf16_round(v)
    return v.reshape(n, hd)


def kv_init(cfg, layers=None) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic committed KV of cfg.ctx positions: arrays [L'][B][Hkv][ctx][hd] (fp32 values)."""
    layers = range(cfg.n_layers) if layers is None else layers
    out = []
    for which in ("k", "v"):
        a = np.empty((len(layers), cfg.batch, cfg.n_kv_heads, cfg.ctx, cfg.head_dim), np.float32)
        for i, l in enumerate(layers):
            for b in range(cfg.batch):
                for g in range(cfg.n_kv_heads):
                    a[i, b, g] = kv_rows(cfg, which, l, b, g, 0, cfg.ctx)
        out.append(a)
    return out[0], out[1]


def state_init(cfg) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic start state: drafter hidden input hid [B][d] (std 1, fp32) and current token t0 [B]."""
    key = stream_key(cfg.state_seed, tensor_id("hid", 0))
    hid = hash_uniform_f32(key, 0, cfg.batch * cfg.d_model, 1.0).reshape(cfg.batch, cfg.d_model)
    tk = stream_key(cfg.state_seed, tensor_id("tok", 0))
    t0 = (hash_u64(tk, 0, cfg.batch) % np.uint64(cfg.vocab)).astype(np.int64)
    return hid, t0


def prompt_tokens(cfg) -> np.ndarray:
    """Prompt of cfg.prompt_len uniform-random token ids per sequence, default_rng(state_seed)."""
    rng = np.random.default_rng(cfg.state_seed)
    return rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.prompt_len)).astype(np.int64)


def inject_key(seed: int, b: int) -> int:
    return stream_key(seed, tensor_id("inject", b))


def inject_threshold(p: float) -> int:
    """Replacement threshold on a 53-bit uniform integer: floor(p * 2^53), clamped to [0, 2^53]."""
    p = min(max(float(p), 0.0), 1.0)
    return int(math.floor(p * float(1 << 53)))


def inject_table(greedy_seq: np.ndarray, K: int, p: float, seed: int, b: int = 0,
                 forced_wrong: bool = False, vocab: int = 0, n_pos: int | None = None) -> np.ndarray:
    """Replacement table for one sequence: entry pos*K + (j-1) is the token that replaces draft
    slot j when it proposes absolute position pos, or -1.  greedy_seq[pos] is the target's own
    greedy token at pos (-1 where unknown).  forced_wrong puts (greedy+1) mod V in every slot."""
    n_pos = len(greedy_seq) if n_pos is None else n_pos
    tab = np.full((n_pos, K), -1, dtype=np.int32)
    g = np.full(n_pos, -1, dtype=np.int64)
    g[: min(n_pos, len(greedy_seq))] = greedy_seq[:n_pos]
    known = g >= 0
    if forced_wrong:
        for j in range(1, K + 1):
            tab[known, j - 1] = (g[known] + 1) % vocab
        return tab.reshape(-1)
    thr = inject_threshold(p)
    pos = np.arange(n_pos, dtype=np.int64)
    key = inject_key(seed, b)
    for j in range(1, K + 1):
        u = hash_u64_at(key, pos * 64 + j) >> np.uint64(11)
        hit = (u < np.uint64(thr)) & known if thr < (1 << 53) else known.copy()
        tab[hit, j - 1] = g[hit]
    return tab.reshape(-1)


def inject_draw(seed: int, b: int, pos: int, j: int) -> int:
    """53-bit uniform integer for draft slot j (1-based) proposing absolute position pos of sequence b."""
    z = int(hash_u64(inject_key(seed, b), pos * 64 + j, 1)[0])
    return z >> 11
