"""Python binding of libspecdec: torch tensors supply device memory and streams, every step of
the path runs in the library's HIP kernels.  No CPU fallback exists: constructing an Engine
without the built library or without a GPU raises."""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _ffi as F

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
ABI_DT = {"bf16": F.BF16, "f32": F.F32}


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _s(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


@dataclass
class Shape:
    """Model shape as the C ABI sees it."""
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    d_layers: int
    d_dim: int
    d_ffn: int
    n_centroids: int
    kv_src_layer: int = -1
    dtype: str = "bf16"
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    shared_ffn: int = 0
    weight_format: str = "dense"  # "dense" (dtype elements) or "q4" (4-bit blocks)

    @classmethod
    def of(cls, cfg) -> "Shape":
        names = cls.__dataclass_fields__.keys()
        return cls(**{n: getattr(cfg, n) for n in names})

    @property
    def q_dim(self):
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim


def pack_matrix(src: torch.Tensor, n: int, kd: int, dtype: str, kind: int = F.PACK_PLAIN,
                head_dim: int = 0, split_rows: int = 0, stream=None) -> torch.Tensor:
    """Packs a logical row-major [n][kd] device matrix into the streaming tile layout."""
    assert src.is_cuda and src.is_contiguous() and src.numel() == n * kd
    dst = torch.empty(n * kd, dtype=src.dtype, device=src.device)
    F.check(F.load().specdec_pack_matrix(_p(src), _p(dst), n, kd, ABI_DT[dtype], kind, head_dim,
                                         split_rows, _s(stream)), "specdec_pack_matrix")
    return dst


def pack_q4(codes: torch.Tensor, steps: torch.Tensor, n: int, kd: int, kind: int = F.PACK_PLAIN,
            head_dim: int = 0, split_rows: int = 0, stream=None) -> torch.Tensor:
    """Packs a logical [n][kd] 4-bit matrix (codes uint8 [n][kd], steps float16 [n][kd/32], device)
    into the library's 4-bit block format."""
    assert codes.is_cuda and codes.is_contiguous() and codes.dtype == torch.uint8
    assert steps.is_cuda and steps.is_contiguous() and steps.dtype == torch.float16
    assert codes.numel() == n * kd and steps.numel() == n * (kd // 32)
    nbytes = F.load().specdec_q4_bytes(n, kd)
    if nbytes == 0:
        raise ValueError(f"no 4-bit layout for [{n}][{kd}]")
    dst = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    F.check(F.load().specdec_pack_q4(_p(codes), _p(steps), _p(dst), n, kd, kind, head_dim,
                                     split_rows, _s(stream)), "specdec_pack_q4")
    return dst


class _Mats:
    """Matrix plumbing for one weight format: a dense matrix is one tensor, a 4-bit one a
    (codes, steps) pair whose parts are concatenated and reindexed together."""

    def __init__(self, source, dtype: str, q4: bool, stream):
        self.source, self.dtype, self.q4, self.stream = source, dtype, q4, stream

    def get(self, name, layer, shape):
        return self.source.get_q4(name, layer, shape) if self.q4 else self.source.get(name, layer, shape)

    def cat(self, parts, dim=0):
        if self.q4:
            return (torch.cat([p[0] for p in parts], dim).contiguous(),
                    torch.cat([p[1] for p in parts], dim).contiguous())
        return torch.cat(parts, dim).contiguous()

    def rows(self, m, index):
        if self.q4:
            return m[0].index_select(0, index).contiguous(), m[1].index_select(0, index).contiguous()
        return m.index_select(0, index).contiguous()

    def pack(self, m, n, kd, kind=F.PACK_PLAIN, head_dim=0, split_rows=0):
        if self.q4:
            return pack_q4(m[0].reshape(-1), m[1].reshape(-1), n, kd, kind, head_dim, split_rows,
                           self.stream)
        return pack_matrix(m.reshape(-1), n, kd, self.dtype, kind, head_dim, split_rows, self.stream)


class DeviceModel:
    """Packed device weights for one target + drafter pair.

    `source.get(name, layer, shape)` must return a logical row-major device tensor of the
    storage dtype (fp32 for norm weights); names follow workloads.synth.TID.  The drafter table is
    stored cluster-major: row r holds vocabulary id perm[r].
    """

    def __init__(self, shape: Shape, source, perm: torch.Tensor, centroids: torch.Tensor,
                 device="cuda", stream=None):
        self.shape = s = shape
        self.device = device
        dt = s.dtype
        keep = self._keep = []

        def k(t):
            keep.append(t)
            return t.data_ptr()

        d, qd, kvd, F_ = s.d_model, s.q_dim, s.kv_dim, s.ffn_dim
        q4 = s.weight_format == "q4"
        if s.weight_format not in ("dense", "q4"):
            raise ValueError(f"weight_format {s.weight_format!r}")
        mm = _Mats(source, dt, q4, stream)
        get, cat, pack = mm.get, mm.cat, mm.pack
        self.layer_ptrs = (C.c_void_p * (s.n_layers * F.N_LAYER_TENSORS))()
        for l in range(s.n_layers):
            qkv = cat([get("wq", l, (qd, d)), get("wk", l, (kvd, d)), get("wv", l, (kvd, d))])
            base = l * F.N_LAYER_TENSORS
            self.layer_ptrs[base + F.LW_QKV] = k(pack(qkv, qd + 2 * kvd, d, F.PACK_ROPE, s.head_dim))
            del qkv
            self.layer_ptrs[base + F.LW_O] = k(pack(get("wo", l, (d, qd)), d, qd))
            if s.n_experts > 0:
                # shared FFN in the dense slots; router and the stacked experts in their own
                E, Fe, Fs = s.n_experts, s.expert_ffn, s.shared_ffn
                names = ("sh_wg", "sh_wu", "sh_wd")
                self.layer_ptrs[base + F.LW_ROUTER] = k(pack(get("router", l, (E, d)), E, d))
                egu = cat([get("exp_wg", l, (E, Fe, d)), get("exp_wu", l, (E, Fe, d))], 1)
                self.layer_ptrs[base + F.LW_EXP_GATE_UP] = k(pack(egu, E * 2 * Fe, d, F.PACK_GATE_UP, split_rows=Fe))
                del egu
                self.layer_ptrs[base + F.LW_EXP_DOWN] = k(pack(get("exp_wd", l, (E, d, Fe)), E * d, Fe))
            else:
                Fs, names = F_, ("wg", "wu", "wd")
            gu = cat([get(names[0], l, (Fs, d)), get(names[1], l, (Fs, d))])
            self.layer_ptrs[base + F.LW_GATE_UP] = k(pack(gu, 2 * Fs, d, F.PACK_GATE_UP, split_rows=Fs))
            del gu
            self.layer_ptrs[base + F.LW_DOWN] = k(pack(get(names[2], l, (d, Fs)), d, Fs))
            self.layer_ptrs[base + F.LW_ATTN_NORM] = k(source.get("attn_norm", l, (d,)).float().contiguous())
            self.layer_ptrs[base + F.LW_FFN_NORM] = k(source.get("ffn_norm", l, (d,)).float().contiguous())
        self.embed = pack(get("embed", 0, (s.vocab, d)), s.vocab, d)
        self.final_norm = source.get("final_norm", 0, (d,)).float().contiguous()

        D, Fd = s.d_dim, s.d_ffn
        perm = perm.to(device=device, dtype=torch.int64)
        table = get("table", 0, (s.vocab, D))
        self.table = pack(mm.rows(table, perm), s.vocab, D)
        del table
        self.row_vocab = perm.to(torch.int32).contiguous()
        inv = torch.empty_like(perm)
        inv[perm] = torch.arange(s.vocab, device=device, dtype=torch.int64)
        self.vocab_row = inv.to(torch.int32).contiguous()
        if q4:
            self.centroids = pack(centroids, s.n_centroids, D)
        else:
            self.centroids = pack(centroids.to(device=device, dtype=TORCH_DT[dt]).contiguous(),
                                  s.n_centroids, D)
        self.norm_h = source.get("norm_h", 0, (d,)).float().contiguous()
        self.norm_e = source.get("norm_e", 0, (D,)).float().contiguous()
        self.w_in = pack(get("w_in", 0, (D, d + D)), D, d + D)
        self.norm_f = source.get("d_nf", 0, (D,)).float().contiguous()
        self.w_back = pack(get("w_back", 0, (d, D)), d, D)
        self.dlayer_ptrs = (C.c_void_p * (s.d_layers * F.N_DRAFT_TENSORS))()
        for l in range(s.d_layers):
            base = l * F.N_DRAFT_TENSORS
            self.dlayer_ptrs[base + F.DW_N1] = k(source.get("d_n1", l, (D,)).float().contiguous())
            self.dlayer_ptrs[base + F.DW_N2] = k(source.get("d_n2", l, (D,)).float().contiguous())
            self.dlayer_ptrs[base + F.DW_Q] = k(pack(get("d_wq", l, (qd, D)), qd, D, F.PACK_ROPE, s.head_dim))
            self.dlayer_ptrs[base + F.DW_O] = k(pack(get("d_wo", l, (D, qd)), D, qd))
            gu = cat([get("d_wg", l, (Fd, D)), get("d_wu", l, (Fd, D))])
            self.dlayer_ptrs[base + F.DW_GATE_UP] = k(pack(gu, 2 * Fd, D, F.PACK_GATE_UP, split_rows=Fd))
            self.dlayer_ptrs[base + F.DW_DOWN] = k(pack(get("d_wd", l, (D, Fd)), D, Fd))

    def abi(self) -> F.Weights:
        w = F.Weights()
        w.embed = self.embed.data_ptr()
        w.final_norm = self.final_norm.data_ptr()
        w.layers = C.cast(self.layer_ptrs, C.POINTER(C.c_void_p))
        w.table = self.table.data_ptr()
        w.centroids = self.centroids.data_ptr()
        w.row_vocab = self.row_vocab.data_ptr()
        w.vocab_row = self.vocab_row.data_ptr()
        w.norm_h = self.norm_h.data_ptr()
        w.norm_e = self.norm_e.data_ptr()
        w.w_in = self.w_in.data_ptr()
        w.d_layers = C.cast(self.dlayer_ptrs, C.POINTER(C.c_void_p))
        w.norm_f = self.norm_f.data_ptr()
        w.w_back = self.w_back.data_ptr()
        return w

    def weight_bytes(self) -> int:
        tot = sum(t.numel() * t.element_size() for t in self._keep)
        for t in (self.embed, self.final_norm, self.table, self.centroids, self.w_in, self.w_back):
            tot += t.numel() * t.element_size()
        return tot


class Engine:
    """One libspecdec context plus the caller-owned device state it works on."""

    def __init__(self, model: DeviceModel, max_batch: int, max_draft: int, max_rows: int,
                 max_ctx: int, stream=None, static_workspace: bool = False, max_prefill: int = 0):
        """static_workspace=True creates the context with specdec_create_static: the library's
        own fixed workspace array instead of a caller buffer (one such context per GPU)."""
        lib = F.load()
        if not torch.cuda.is_available():
            raise RuntimeError("libspecdec needs a ROCm GPU; no CPU path exists")
        s = model.shape
        self.model = model
        self.shape = s
        self.lib = lib
        cfg = F.Config()
        for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
                  "n_experts", "top_k", "expert_ffn", "shared_ffn", "d_layers", "d_dim", "d_ffn",
                  "n_centroids", "kv_src_layer"):
            setattr(cfg, n, int(getattr(s, n)))
        cfg.dtype = ABI_DT[s.dtype]
        cfg.rms_eps = s.rms_eps
        cfg.rope_theta = s.rope_theta
        cfg.max_batch, cfg.max_draft, cfg.max_rows, cfg.max_ctx = max_batch, max_draft, max_rows, max_ctx
        cfg.weight_format = F.WF_Q4 if s.weight_format == "q4" else F.WF_DENSE
        cfg.max_prefill = max_prefill
        self.cfg = cfg
        self.max_batch, self.max_draft, self.max_rows, self.max_ctx = max_batch, max_draft, max_rows, max_ctx
        ws = lib.specdec_workspace_bytes(C.byref(cfg))
        if ws == 0:
            raise F.SpecdecError(F.E_INVAL, "specdec_workspace_bytes (invalid configuration)")
        dev = model.device
        kv = lib.specdec_kv_elems(C.byref(cfg))
        self.kv_k = torch.zeros(kv, dtype=TORCH_DT[s.dtype], device=dev)
        self.kv_v = torch.zeros(kv, dtype=TORCH_DT[s.dtype], device=dev)
        self.len = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.hid = torch.zeros(max_batch, s.d_model, dtype=torch.float32, device=dev)
        self.ws_bytes = ws
        self._w = model.abi()
        ctx = C.c_void_p()
        if static_workspace:
            self._ws = None
            F.check(lib.specdec_create_static(C.byref(cfg), C.byref(self._w), _p(self.kv_k),
                                              _p(self.kv_v), _p(self.len), _p(self.hid),
                                              _s(stream), C.byref(ctx)), "specdec_create_static")
        else:
            self._ws = torch.zeros(ws + 256, dtype=torch.uint8, device=dev)
            off = (-self._ws.data_ptr()) % 256
            self.ws_ptr = self._ws.data_ptr() + off
            F.check(lib.specdec_create(C.byref(cfg), C.byref(self._w), _p(self.kv_k),
                                       _p(self.kv_v), _p(self.len), _p(self.hid),
                                       C.c_void_p(self.ws_ptr), ws, _s(stream), C.byref(ctx)),
                    "specdec_create")
        self.ctx = ctx

    # --- state helpers (setup / tests) ---
    def kv_view(self):
        """K as [L][B][Hkv][max_ctx][hd] and V as [L][B][Hkv][hd][max_ctx]."""
        s = self.shape
        shp = (s.n_layers, self.max_batch, s.n_kv_heads, self.max_ctx, s.head_dim)
        vshp = (s.n_layers, self.max_batch, s.n_kv_heads, s.head_dim, self.max_ctx)
        return self.kv_k.view(shp), self.kv_v.view(vshp)

    def set_len(self, values) -> None:
        vals = [int(v) for v in values]
        self.len[: len(vals)].copy_(torch.tensor(vals, dtype=torch.int32))
        self.set_len_bound(vals)

    def set_len_bound(self, values) -> None:
        arr = (C.c_int32 * len(values))(*[int(v) for v in values])
        F.check(self.lib.specdec_set_len_bound(self.ctx, arr, len(values)), "specdec_set_len_bound")

    def device_error(self, clear: bool = True, stream=None) -> int:
        w = C.c_int32()
        F.check(self.lib.specdec_read_device_error(self.ctx, C.byref(w), int(clear), _s(stream)),
                "specdec_read_device_error")
        return int(w.value)

    # --- the four step calls ---
    def verify(self, tokens, logits=None, argmax=None, stream=None) -> None:
        B, R = tokens.shape
        F.check(self.lib.specdec_verify(self.ctx, B, R, _p(tokens), _p(logits), _p(argmax),
                                        _s(stream)), "specdec_verify")

    def prefill(self, b: int, tokens, logits=None, argmax=None, stream=None) -> None:
        """Runs the prompt chunk tokens (int32 [T], device) of sequence b through the target and
        commits it (specdec_prefill)."""
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        F.check(self.lib.specdec_prefill(self.ctx, b, tokens.numel(), _p(tokens), _p(logits),
                                         _p(argmax), _s(stream)), "specdec_prefill")

    def accept(self, tokens, out_tokens=None, n_emit=None, next_tok=None, commit=True,
               stream=None) -> None:
        B, R = tokens.shape
        F.check(self.lib.specdec_accept(self.ctx, B, R - 1, _p(tokens), _p(out_tokens), _p(n_emit),
                                        _p(next_tok), F.ACCEPT_COMMIT if commit else 0, _s(stream)),
                "specdec_accept")

    def kv_commit(self, n_commit, stream=None) -> None:
        F.check(self.lib.specdec_kv_commit(self.ctx, n_commit.shape[0], _p(n_commit), _s(stream)),
                "specdec_kv_commit")

    def draft(self, cur_tok, drafts, head_mode=F.HEAD_CLUSTERED, k_c=1, inject=None,
              verify_tokens=None, trace=None, stream=None) -> None:
        """Drafts [B][K] from cur_tok [B]; optionally also writes the verify input rows
        verify_tokens [B][K+1] = [cur, d1..dK] (after injection).  `trace`, a dict with any of
        the keys state [B][K][d_dim], hidden [B][K][d_model], centroid_scores [B][K][Nc],
        table_scores [B][K][V] (float32) and raw_drafts [B][K] (int32), receives the drafter's
        intermediate values (specdec_draft_traced)."""
        B, K = drafts.shape
        if verify_tokens is not None:
            assert verify_tokens.is_contiguous() and tuple(verify_tokens.shape) == (B, K + 1)
        stride = 0 if inject is None else inject.shape[1]
        if trace is None:
            F.check(self.lib.specdec_draft(self.ctx, B, K, head_mode, k_c, _p(cur_tok), _p(drafts),
                                           _p(inject), stride, _p(verify_tokens), _s(stream)),
                    "specdec_draft")
            return
        s = self.shape
        widths = {"state": s.d_dim, "hidden": s.d_model, "centroid_scores": s.n_centroids,
                  "table_scores": s.vocab, "raw_drafts": 1}
        tr = F.DraftTrace()
        for name, t in trace.items():
            want = (torch.int32 if name == "raw_drafts" else torch.float32)
            assert t.is_contiguous() and t.dtype == want and t.numel() == B * K * widths[name], name
            setattr(tr, name, t.data_ptr())
        F.check(self.lib.specdec_draft_traced(self.ctx, B, K, head_mode, k_c, _p(cur_tok),
                                              _p(drafts), _p(inject), stride, _p(verify_tokens),
                                              C.byref(tr), _s(stream)), "specdec_draft_traced")

    # --- token trees ---
    @staticmethod
    def _parents(parent):
        return (C.c_int32 * len(parent))(*[int(v) for v in parent])

    def draft_tree(self, cur_tok, tree_tokens, width: int, depth: int, head_mode=F.HEAD_CLUSTERED,
                   k_c=1, inject=None, stream=None) -> None:
        """A width x depth tree draft into tree_tokens [B][1 + width*depth] (node order)."""
        B = tree_tokens.shape[0]
        assert tree_tokens.is_contiguous() and tree_tokens.shape[1] == 1 + width * depth
        stride = 0 if inject is None else inject.shape[1]
        F.check(self.lib.specdec_draft_tree(self.ctx, B, width, depth, head_mode, k_c, _p(cur_tok),
                                            _p(tree_tokens), _p(inject), stride, _s(stream)),
                "specdec_draft_tree")

    def verify_tree(self, parent, tokens, logits=None, argmax=None, stream=None) -> None:
        B, n = tokens.shape
        F.check(self.lib.specdec_verify_tree(self.ctx, B, n, self._parents(parent), _p(tokens),
                                             _p(logits), _p(argmax), _s(stream)), "specdec_verify_tree")

    def accept_tree(self, parent, tokens, out_tokens, n_emit=None, next_tok=None, commit=True,
                    stream=None) -> None:
        B, n = tokens.shape
        F.check(self.lib.specdec_accept_tree(self.ctx, B, n, self._parents(parent), _p(tokens),
                                             _p(out_tokens), out_tokens.shape[1], _p(n_emit),
                                             _p(next_tok), F.ACCEPT_COMMIT if commit else 0,
                                             _s(stream)), "specdec_accept_tree")

    def moe_usage_start(self, stream=None) -> None:
        F.check(self.lib.specdec_moe_usage_start(self.ctx, _s(stream)), "specdec_moe_usage_start")

    def moe_usage_read(self, stream=None) -> list:
        """Per layer, the summed number of distinct experts routed to since moe_usage_start."""
        n = self.shape.n_layers
        buf = (C.c_int32 * n)()
        F.check(self.lib.specdec_moe_usage_read(self.ctx, buf, _s(stream)), "specdec_moe_usage_read")
        return [buf[i] for i in range(n)]

    # --- measurement helpers ---
    def profile_start(self, kernel_class: int, capacity: int) -> None:
        F.check(self.lib.specdec_profile_start(self.ctx, kernel_class, capacity), "specdec_profile_start")

    def profile_read(self, max_n: int = 100000) -> list:
        buf = (C.c_float * max_n)()
        n = C.c_int32()
        F.check(self.lib.specdec_profile_read(self.ctx, buf, max_n, C.byref(n)), "specdec_profile_read")
        return [buf[i] for i in range(n.value)]

    def query_split(self, kernel_class: int):
        """(split-K factor, work units, waves per workgroup, workgroups) of one launch."""
        s, u, w, g = C.c_int32(), C.c_int32(), C.c_int32(), C.c_int32()
        F.check(self.lib.specdec_query_split(self.ctx, kernel_class, C.byref(s), C.byref(u),
                                             C.byref(w), C.byref(g)), "specdec_query_split")
        return s.value, u.value, w.value, g.value

    def query_launch(self, kernel_class: int, rows: int):
        """(split-K factor, tiles per unit, work units, waves per workgroup, workgroups) of one
        launch of a call of `rows` rows."""
        v = [C.c_int32() for _ in range(5)]
        F.check(self.lib.specdec_query_launch(self.ctx, kernel_class, rows,
                                              *[C.byref(x) for x in v]), "specdec_query_launch")
        return tuple(x.value for x in v)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self.lib.specdec_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tree_parents(width: int, depth: int) -> list:
    """Parent of every node of the tree specdec_draft_tree writes (node order: the root, then
    level by level, branch k at node 1 + width*(j-1) + k)."""
    return [-1] + [0 if j == 1 else 1 + width * (j - 2) + k
                   for j in range(1, depth + 1) for k in range(width)]


class KPolicy:
    """The library's draft-length policy (specdec_k_policy_*): host code, no device work."""

    def __init__(self, k_min: int, k_max: int, t_draft_ms: float, t_verify_ms: float,
                 t_row_ms: float, decay: float = 0.9, prior_accepted: float = 1.0,
                 prior_rejected: float = 1.0):
        self.lib = F.load()
        self.s = F.KPolicy()
        F.check(self.lib.specdec_k_policy_init(C.byref(self.s), k_min, k_max, decay,
                                               prior_accepted, prior_rejected, t_draft_ms,
                                               t_verify_ms, t_row_ms), "specdec_k_policy_init")

    def observe(self, K: int, n_emit) -> None:
        arr = (C.c_int32 * len(n_emit))(*[int(n) for n in n_emit])
        F.check(self.lib.specdec_k_policy_observe(C.byref(self.s), K, arr, len(n_emit)),
                "specdec_k_policy_observe")

    def acceptance(self) -> float:
        return float(self.lib.specdec_k_policy_acceptance(C.byref(self.s)))

    def choose(self) -> int:
        k = int(self.lib.specdec_k_policy_choose(C.byref(self.s)))
        if k < 0:
            F.check(k, "specdec_k_policy_choose")
        return k
