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
                 weights_override=None, max_prefill: int = 0):
    src = source or WD.source_for(cfg)
    if weights_override is not None:
        src = weights_override(src)
    perm, cent = WD.clusters(cfg)
    model = E.DeviceModel(E.Shape.of(cfg), src, perm, cent)
    eng = E.Engine(model, max_batch=max_batch, max_draft=max(cfg.draft_k, 1),
                   max_rows=max(max_rows, cfg.draft_k + 1), max_ctx=max_ctx,
                   max_prefill=max_prefill)
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


def gpu_greedy_margins(eng, t0: int, n: int):
    """gpu_greedy that also returns each step's top-2 logit margin (from the GPU's own logits)."""
    dev = eng.kv_k.device
    V = eng.shape.vocab
    toks, margins = [int(t0)], []
    cur = torch.tensor([[t0]], dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    lg = torch.empty(1, 1, V, dtype=torch.float32, device=dev)
    while len(toks) < n:
        eng.verify(cur, logits=lg)
        eng.accept(cur, next_tok=nxt, commit=True)
        top2 = torch.topk(lg[0, 0], 2).values
        margins.append(float(top2[0] - top2[1]))
        cur = nxt.view(1, 1).clone()
        toks.append(int(nxt.item()))
    return toks, margins


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


def host_embedding(cfg) -> np.ndarray:
    """The tied embedding / LM head [V][d] as float32 on the host, made by the device fill of the
    seeded input generator (bit-identical to the host generator, spot-checked here).  4-bit
    weights are turned into values by the oracle's q4_weights, in row blocks (exact in fp32)."""
    src = WD.DeviceSource(cfg)
    shape = (cfg.vocab, cfg.d_model)
    if cfg.weight_format == "q4":
        codes, steps = src.get_q4("embed", 0, shape)
        E = np.empty(shape, dtype=np.float32)
        for r0 in range(0, cfg.vocab, 16384):
            c = codes[r0:r0 + 16384].cpu().numpy()
            d = steps[r0:r0 + 16384].cpu().numpy()
            E[r0:r0 + 16384] = O.q4_weights(c, d)
        del codes, steps
    else:
        t = src.get("embed", 0, shape)
        E = t.float().cpu().numpy()
        del t
    for r in (0, 12345 % cfg.vocab, cfg.vocab - 1):
        assert np.array_equal(E[r], O.as_f64(S.gen_rows(cfg, "embed", 0, cfg.d_model, r, 1))[0])
    return E


def oracle_logits_full(cfg, W, E32, hs, chunk: int = 32768) -> np.ndarray:
    """The oracle's LM head over the whole vocabulary for each hidden row in hs, applied to row
    blocks of the embedding E32 (float32 values of the storage type)."""
    out = np.empty((len(hs), cfg.vocab))
    if len(hs) == 0:
        return out
    X = np.stack(hs)
    for r0 in range(0, cfg.vocab, chunk):
        blk = {"embed": E32[r0:r0 + chunk].astype(np.float64), "final_norm": W["final_norm"]}
        out[:, r0:r0 + chunk] = O.lm_head(blk, cfg, X)
    return out


def drafter_trace_check(eng, cfg, DW, cache, hid, t0: int, length: int, K: int, mode: str,
                        k_c: int, tol: float, margin: float = 0.05):
    """Runs one traced draft of K sub-steps and checks every sub-step against the oracle,
    teacher-forced on the GPU's own tokens (sub-step j of the oracle reads the token the GPU
    drafted at j-1, so a legitimate near-tie flip does not end the comparison):

    * the head's input s, the next hidden W_back s and (clustered) the centroid scores, element by
      element within `tol` (max relative error);
    * the clusters the GPU scored are exactly the k_c best of its own centroid scores (ties ->
      lower cluster id), and its token is the argmax of its own scores over those members (ties
      -> lower vocabulary id): bit-exact integer decisions taken from the GPU's values;
    * the GPU's token scores within `tol` of the oracle's at every scored row;
    * where the oracle's own choice differs, a near tie explains it: a cluster the GPU took over
      the oracle's choice scores within tol * max|z| of the oracle's k_c-th best, or (same
      clusters) the two tokens' oracle scores are within `margin`.

    Returns the list of sub-steps at which the oracle's token differed (near ties)."""
    dev = eng.kv_k.device
    s = eng.shape
    V, Nc, S = s.vocab, s.n_centroids, s.vocab // s.n_centroids
    drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
    tr = {"state": torch.empty(1, K, s.d_dim, dtype=torch.float32, device=dev),
          "hidden": torch.empty(1, K, s.d_model, dtype=torch.float32, device=dev),
          "table_scores": torch.full((1, K, V), float("nan"), dtype=torch.float32, device=dev),
          "raw_drafts": torch.empty(1, K, dtype=torch.int32, device=dev)}
    if mode == "clustered":
        tr["centroid_scores"] = torch.empty(1, K, Nc, dtype=torch.float32, device=dev)
    hm = SD.HEAD_FULL if mode == "full" else SD.HEAD_CLUSTERED
    eng.draft(torch.tensor([t0], dtype=torch.int32, device=dev), drafts, head_mode=hm, k_c=k_c,
              trace=tr)
    got = {k: v[0].cpu().numpy() for k, v in tr.items()}
    raw = got["raw_drafts"].tolist()
    assert drafts[0].cpu().tolist() == raw, "without injection the drafts are the drafter's own"
    perm = np.asarray(DW["perm"])
    h, c, flips = np.asarray(hid, np.float64), int(t0), []
    for j in range(K):
        st = []
        d_ref, h_next = O.drafter_substep(DW, cfg, cache, h, c, length + j, length, mode, k_c, st)
        s_ref = st[0]
        assert rel_err(got["state"][j], s_ref) < tol, f"sub-step {j + 1}: head input s"
        assert rel_err(got["hidden"][j], h_next) < tol, f"sub-step {j + 1}: next hidden"
        sc = got["table_scores"][j]
        rows = np.nonzero(~np.isnan(sc))[0]
        if mode == "clustered":
            gz = got["centroid_scores"][j]
            z_ref = O.centroid_scores(DW["centroids"], s_ref)
            assert rel_err(gz, z_ref) < tol, f"sub-step {j + 1}: centroid scores"
            sel = sorted(range(Nc), key=lambda q: (-float(gz[q]), q))[:k_c]
            want = np.sort(np.concatenate([np.arange(q * S, (q + 1) * S) for q in sel]))
            assert np.array_equal(rows, want), f"sub-step {j + 1}: scored rows are not the GPU's best clusters"
        else:
            assert len(rows) == V, f"sub-step {j + 1}: the full head left rows unscored"
        ids = perm[rows]  # table row r holds vocabulary id perm[r]
        vals = sc[rows]
        best = float(vals.max())
        assert raw[j] == int(ids[vals == best].min()), f"sub-step {j + 1}: not the argmax of its own scores"
        ref_sc = O.token_scores(DW["table"][ids], s_ref)
        assert rel_err(vals, ref_sc) < tol, f"sub-step {j + 1}: token scores"
        if d_ref != raw[j]:
            flips.append(j + 1)
            if mode == "clustered":
                z_ref = O.centroid_scores(DW["centroids"], s_ref)
                osel = sorted(range(Nc), key=lambda q: (-z_ref[q], q))[:k_c]
                if set(osel) != set(sel):
                    kth = float(np.sort(z_ref)[::-1][k_c - 1])
                    delta = tol * float(np.max(np.abs(z_ref)))
                    assert all(z_ref[q] >= kth - delta for q in sel), f"sub-step {j + 1}: cluster choice"
                    h, c = h_next, raw[j]
                    continue
            full_ref = O.token_scores(DW["table"], s_ref)
            assert full_ref[d_ref] - full_ref[raw[j]] <= margin, f"sub-step {j + 1}: token choice"
        h, c = h_next, raw[j]
    assert eng.device_error() == 0
    return flips


def gpu_spec_tree(eng, t0: int, n: int, width: int, depth: int, inject_tab=None,
                  head_mode=SD.HEAD_CLUSTERED, k_c=1):
    """The speculative loop with tree drafts through the C ABI; returns (tokens, emitted per
    step)."""
    dev = eng.kv_k.device
    par = E.tree_parents(width, depth)
    nn = len(par)
    toks = [int(t0)]
    cur = torch.tensor([t0], dtype=torch.int32, device=dev)
    T = torch.empty(1, nn, dtype=torch.int32, device=dev)
    out = torch.empty(1, depth + 1, dtype=torch.int32, device=dev)
    n_emit = torch.empty(1, dtype=torch.int32, device=dev)
    inj = None if inject_tab is None else torch.from_numpy(inject_tab.reshape(1, -1)).to(dev)
    emitted = []
    length = int(eng.len[0].item())
    while len(toks) < n:
        eng.draft_tree(cur, T, width, depth, head_mode=head_mode, k_c=k_c, inject=inj)
        eng.verify_tree(par, T)
        eng.accept_tree(par, T, out, n_emit=n_emit, next_tok=cur, commit=True)
        e = int(n_emit.item())
        toks.extend(out[0, :e].cpu().tolist())
        emitted.append(e)
        length += e
        eng.set_len_bound([length])
    return toks[:n], emitted
