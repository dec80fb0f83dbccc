"""Helpers for the GPU parity tests: build an engine for a workload, run prefill / greedy / the
speculative loop through the C ABI, and compare against the oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
import speculative_decoding_03_amd as SD
from speculative_decoding_03_amd import engine as E
from workloads import device as WD
from workloads import synth as S


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    """max |a - ref| / max |ref| (per row: caller passes one row)."""
    return float(np.max(np.abs(a.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def build_engine(cfg, max_ctx: int, max_rows: int = 16, max_batch: int = 1, source=None,
                 weights_override=None):
    src = source or WD.source_for(cfg)
    if weights_override is not None:
        src = weights_override(src)
    perm, cent = WD.clusters(cfg)
    model = E.DeviceModel(E.Shape.of(cfg), src, perm, cent)
    eng = E.Engine(model, max_batch=max_batch, max_draft=max(cfg.draft_k, 1),
                   max_rows=max(max_rows, cfg.draft_k + 1), max_ctx=max_ctx)
    return eng


def gpu_prefill(eng, prompt: np.ndarray, chunk: int = 16, want_logits: bool = True):
    """verify(chunk) + kv_commit(chunk) over the prompt; returns (first token, logits rows)."""
    dev = eng.kv_k.device
    V = eng.shape.vocab
    rows = []
    am = None
    for s in range(0, len(prompt), chunk):
        part = prompt[s:s + chunk]
        toks = torch.tensor(part, dtype=torch.int32, device=dev).view(1, -1)
        lg = torch.empty(1, len(part), V, dtype=torch.float32, device=dev) if want_logits else None
        am = torch.empty(1, len(part), dtype=torch.int32, device=dev)
        eng.verify(toks, logits=lg, argmax=am)
        eng.kv_commit(torch.tensor([len(part)], dtype=torch.int32, device=dev))
        if want_logits:
            rows.append(lg[0].cpu().numpy())
    eng.set_len_bound([len(prompt)])
    return int(am[0, -1].item()), (np.concatenate(rows) if want_logits else None)


def gpu_greedy(eng, t0: int, n: int):
    """Plain greedy decoding through verify(1 row) + accept(K=0, commit).  Returns n tokens
    (t0 first), including each step's logits row."""
    dev = eng.kv_k.device
    toks = [int(t0)]
    cur = torch.tensor([[t0]], dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    while len(toks) < n:
        eng.verify(cur)
        eng.accept(cur, next_tok=nxt, commit=True)
        cur = nxt.view(1, 1).clone()
        toks.append(int(nxt.item()))
    return toks


def gpu_spec(eng, t0: int, n: int, K: int, inject_tab=None, head_mode=SD.HEAD_CLUSTERED, k_c=1):
    """The speculative loop through the C ABI; returns (tokens, emitted per step)."""
    dev = eng.kv_k.device
    toks = [int(t0)]
    cur = torch.tensor([t0], dtype=torch.int32, device=dev)
    drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
    out = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    n_emit = torch.empty(1, dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    inj = None if inject_tab is None else torch.from_numpy(inject_tab.reshape(1, -1)).to(dev)
    emitted = []
    length = int(eng.len[0].item())
    while len(toks) < n:
        eng.draft(cur, drafts, head_mode=head_mode, k_c=k_c, inject=inj)
        T = torch.cat([cur.view(1, 1), drafts], 1).contiguous()
        eng.verify(T)
        eng.accept(T, out_tokens=out, n_emit=n_emit, next_tok=nxt, commit=True)
        e = int(n_emit.item())
        toks.extend(out[0, :e].cpu().tolist())
        emitted.append(e)
        length += e
        eng.set_len_bound([length])  # the host now knows the committed length exactly
        cur = nxt.clone()
    return toks[:n], emitted


def gpu_prefill_batch(eng, prompts: np.ndarray, chunk: int = 16):
    """verify(chunk) + kv_commit(chunk) over B equal-length prompts [B][L]; returns the first
    generated token of each sequence."""
    dev = eng.kv_k.device
    B, L = prompts.shape
    am = None
    for s in range(0, L, chunk):
        part = torch.tensor(prompts[:, s:s + chunk], dtype=torch.int32, device=dev).contiguous()
        am = torch.empty(B, part.shape[1], dtype=torch.int32, device=dev)
        eng.verify(part, argmax=am)
        eng.kv_commit(torch.full((B,), part.shape[1], dtype=torch.int32, device=dev))
    eng.set_len_bound([L] * B)
    return am[:, -1].cpu().tolist()


def gpu_greedy_batch(eng, t0s, n: int):
    """Plain greedy decoding of B sequences at once (verify of one row each + accept)."""
    dev = eng.kv_k.device
    B = len(t0s)
    cur = torch.tensor(t0s, dtype=torch.int32, device=dev).view(B, 1)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    toks = [[int(t)] for t in t0s]
    while len(toks[0]) < n:
        eng.verify(cur)
        eng.accept(cur, next_tok=nxt, commit=True)
        cur = nxt.view(B, 1).clone()
        for b, t in enumerate(nxt.cpu().tolist()):
            toks[b].append(t)
    return toks


def gpu_spec_batch(eng, t0s, n: int, K: int, inject_tabs: np.ndarray):
    """The speculative loop over B sequences at once, the draft writing the verify rows."""
    dev = eng.kv_k.device
    B = len(t0s)
    cur = torch.tensor(t0s, dtype=torch.int32, device=dev)
    drafts = torch.empty(B, K, dtype=torch.int32, device=dev)
    T = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    out = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    n_emit = torch.empty(B, dtype=torch.int32, device=dev)
    inj = torch.from_numpy(np.ascontiguousarray(inject_tabs)).to(dev)
    toks = [[int(t)] for t in t0s]
    lengths = eng.len[:B].cpu().tolist()
    emitted = []
    while min(len(t) for t in toks) < n:
        eng.draft(cur, drafts, inject=inj, verify_tokens=T)
        eng.verify(T)
        eng.accept(T, out_tokens=out, n_emit=n_emit, next_tok=cur, commit=True)
        e = n_emit.cpu().tolist()
        o = out.cpu().tolist()
        for b in range(B):
            toks[b].extend(o[b][: e[b]])
            lengths[b] += e[b]
        emitted.append(e)
        eng.set_len_bound(lengths)
    return [t[:n] for t in toks], emitted


def snapshot(eng):
    return eng.len.clone(), eng.hid.clone()


def restore(eng, snap):
    ln, hid = snap
    eng.len.copy_(ln)
    eng.hid.copy_(hid)
    eng.set_len_bound(ln.cpu().tolist())


def oracle_model(cfg):
    return O.as_f64(S.target_weights(cfg)), O.as_f64(S.drafter_weights(cfg))
