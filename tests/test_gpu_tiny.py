"""GPU parity on the tiny fp32 workloads (2 layers, d=256, vocab 4096, drafter d=128 with 64
centroids of 64 tokens; prompt 64 ids; 64 generated tokens; K=3), through the C ABI: the dense
target and its mixture-of-experts twin (16 experts of FFN 128, top-4, shared FFN 256).

Tolerance: logits within a max relative error of 1e-4 (fp32); tokens must match wherever the
oracle's top-2 logit margin exceeds 0.05; acceptance and indexing bit-exact given logits."""

import itertools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle as O  # noqa: E402
import speculative_decoding_03_amd as SD  # noqa: E402
from gpu_util import (build_engine, drafter_trace_check, gpu_greedy, gpu_greedy_batch,  # noqa: E402
                      gpu_prefill, gpu_prefill_batch, gpu_spec, gpu_spec_batch, oracle_model,
                      rel_err, restore, snapshot)
from workloads import inject_table, preset, prompt_tokens  # noqa: E402

CFG = preset("tiny")
MAX_CTX = 256
TOL = 1e-4


@pytest.fixture(scope="module", params=["tiny", "tiny-moe"])
def tiny(request):
    """GPU engine after prefill, plus the oracle's state after the same prefill."""
    CFG = preset(request.param)
    eng = build_engine(CFG, MAX_CTX)
    prompt = prompt_tokens(CFG)[0]
    t0, logits = gpu_prefill(eng, prompt)
    W, DW = oracle_model(CFG)
    cache = O.KVCache.empty(CFG, MAX_CTX)
    ref_rows = []
    lg = hidden = None
    for pos, tok in enumerate(prompt):
        lg, hidden = O.target_row(W, CFG, cache, int(tok), pos)
        ref_rows.append(lg)
    ref_t0 = O.argmax_first(lg)
    n = CFG.gen_tokens
    K = CFG.draft_k
    greedy, margins = O.greedy_generate(W, CFG, cache.copy(), ref_t0, len(prompt), n + K + 2,
                                        record_margins=True)
    yield dict(cfg=CFG, eng=eng, t0=t0, logits=logits, ref_rows=np.array(ref_rows), ref_t0=ref_t0,
                W=W, DW=DW, cache=cache, hid=hidden, length=len(prompt), greedy=greedy,
                margins=margins, snap=snapshot(eng))
    eng.close()


def test_prefill_logits_match_oracle(tiny):
    CFG = tiny["cfg"]
    errs = [rel_err(tiny["logits"][i], tiny["ref_rows"][i]) for i in range(len(tiny["ref_rows"]))]
    assert max(errs) < TOL, f"max rel err {max(errs):.3e}"
    assert tiny["t0"] == tiny["ref_t0"]
    eng = tiny["eng"]
    assert int(eng.len[0].item()) == tiny["length"]
    assert rel_err(eng.hid[0].cpu().numpy(), tiny["hid"]) < TOL
    assert eng.device_error() == 0


def test_prefill_in_calls_of_32_rows(tiny):
    """Prefill in 32-row verify calls: 64 query vectors per KV head, more than the attention
    kernel stages in LDS (32), so it reads each 16-vector tile's queries from global memory."""
    CFG = tiny["cfg"]
    eng = build_engine(CFG, MAX_CTX, max_rows=32)
    try:
        prompt = prompt_tokens(CFG)[0]
        t0, logits = gpu_prefill(eng, prompt, chunk=32)
        errs = [rel_err(logits[i], tiny["ref_rows"][i]) for i in range(len(tiny["ref_rows"]))]
        assert max(errs) < TOL, f"max rel err {max(errs):.3e}"
        assert t0 == tiny["ref_t0"]
        assert eng.device_error() == 0
    finally:
        eng.close()


def _check_tokens(gpu_toks, ref_toks, margins, n):
    """Tokens must match wherever the oracle's margin exceeds 0.05; stop at an allowed flip."""
    for i in range(1, n):
        if gpu_toks[i] != ref_toks[i]:
            assert margins[i - 1] <= 0.05, f"token {i} differs at margin {margins[i - 1]:.4f}"
            return i
    return n


def test_gpu_greedy_matches_oracle(tiny):
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    restore(eng, tiny["snap"])
    n = CFG.gen_tokens
    toks = gpu_greedy(eng, tiny["t0"], n)
    _check_tokens(toks, tiny["greedy"], tiny["margins"], n)
    tiny["gpu_greedy"] = toks
    assert eng.device_error() == 0


@pytest.mark.parametrize("p", [0.0, 0.6, 1.0, "wrong"])
def test_gpu_spec_equals_gpu_greedy(tiny, p):
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    n, K = CFG.gen_tokens, CFG.draft_k
    restore(eng, tiny["snap"])
    ref = gpu_greedy(eng, tiny["t0"], n + K + 2)
    restore(eng, tiny["snap"])
    L = tiny["length"]
    gseq = np.full(MAX_CTX, -1, dtype=np.int64)
    gseq[L:L + len(ref)] = ref
    if p == "wrong":
        tab = inject_table(gseq, K, 0.0, CFG.inject_seed, forced_wrong=True, vocab=CFG.vocab)
    else:
        tab = inject_table(gseq, K, p, CFG.inject_seed)
    toks, emitted = gpu_spec(eng, tiny["t0"], n, K, tab)
    assert toks == ref[:n], "speculative output differs from the same GPU's greedy output"
    assert all(1 <= e <= K + 1 for e in emitted)
    if p == 1.0:
        assert all(e == K + 1 for e in emitted)
    if p == "wrong":
        assert all(e == 1 for e in emitted)
    _check_tokens(toks, tiny["greedy"], tiny["margins"], n)
    assert eng.device_error() == 0


@pytest.mark.parametrize("name", ["tiny", "tiny-moe"])
def test_spec_equals_greedy_at_every_draft_length(name):
    """The draft length is a per-call knob: K = 1 (the smallest speculative step: one draft, two
    verify rows), 2 and 5 (past the configured 3) reproduce the same GPU's greedy output, with
    exactly K+1 tokens per step when every draft is the target's own token."""
    cfg = preset(name)
    kmax = 5
    eng = build_engine(cfg.replace(draft_k=kmax), MAX_CTX)
    prompt = prompt_tokens(cfg)[0]
    t0, _ = gpu_prefill(eng, prompt, want_logits=False)
    snap = snapshot(eng)
    n = cfg.gen_tokens
    ref = gpu_greedy(eng, t0, n + kmax + 2)
    L = len(prompt)
    gseq = np.full(MAX_CTX, -1, dtype=np.int64)
    gseq[L:L + len(ref)] = ref
    for K in (1, 2, 5):
        for p in (0.6, 1.0):
            restore(eng, snap)
            toks, emitted = gpu_spec(eng, t0, n, K, inject_table(gseq, K, p, cfg.inject_seed))
            assert toks == ref[:n], f"K={K} p={p}"
            assert all(1 <= e <= K + 1 for e in emitted)
            if p == 1.0:
                assert all(e == K + 1 for e in emitted), f"K={K}"
    assert eng.device_error() == 0
    eng.close()


@pytest.mark.parametrize("p", [0.0, 0.6, 1.0])
def test_adaptive_draft_length_reproduces_greedy(tiny, p):
    """Speculative steps whose draft length the library's policy picks from the running
    acceptance (K between 1 and 6, changing step to step) reproduce the same GPU's greedy
    output; at p = 1 the policy climbs to the longest draft, at p = 0 it stays at the shortest."""
    CFG = tiny["cfg"]
    eng = build_engine(CFG.replace(draft_k=6), MAX_CTX)
    try:
        prompt = prompt_tokens(CFG)[0]
        t0, _ = gpu_prefill(eng, prompt, want_logits=False)
        n, kmax = 48, 6
        L = len(prompt)
        snap = snapshot(eng)
        ref = gpu_greedy(eng, t0, n + kmax + 2)
        restore(eng, snap)
        gseq = np.full(MAX_CTX, -1, dtype=np.int64)
        gseq[L:L + len(ref)] = ref
        dev = eng.kv_k.device
        tabs = {K: torch.from_numpy(inject_table(gseq, K, p, CFG.inject_seed).reshape(1, -1)).to(dev)
                for K in range(1, kmax + 1)}
        pol = SD.KPolicy(1, kmax, t_draft_ms=0.05, t_verify_ms=1.0, t_row_ms=0.02, decay=0.8)
        cur = torch.tensor([t0], dtype=torch.int32, device=dev)
        toks, ks = [t0], []
        while len(toks) < n:
            K = pol.choose()
            ks.append(K)
            drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
            T = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
            out = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
            n_emit = torch.empty(1, dtype=torch.int32, device=dev)
            eng.draft(cur, drafts, inject=tabs[K], verify_tokens=T)
            eng.verify(T)
            eng.accept(T, out_tokens=out, n_emit=n_emit, next_tok=cur, commit=True)
            e = int(n_emit.item())
            pol.observe(K, [e])
            toks.extend(out[0, :e].cpu().tolist())
            eng.set_len_bound([int(eng.len[0].item())])
        assert toks[:n] == ref[:n]
        if p == 1.0:
            assert ks[-1] == kmax
        if p == 0.0:
            assert ks[-1] == 1
        assert len(set(ks)) > 1 or p == 0.0
        assert eng.device_error() == 0
    finally:
        eng.close()


@pytest.mark.parametrize("mode,k_c", [("clustered", 1), ("clustered", 3), ("clustered", 64), ("full", 0)])
def test_drafter_matches_oracle(tiny, mode, k_c):
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    restore(eng, tiny["snap"])
    K = CFG.draft_k
    dev = eng.kv_k.device
    cur = torch.tensor([tiny["t0"]], dtype=torch.int32, device=dev)
    drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
    hm = SD.HEAD_FULL if mode == "full" else SD.HEAD_CLUSTERED
    eng.draft(cur, drafts, head_mode=hm, k_c=max(k_c, 1))
    got = drafts[0].cpu().tolist()
    ref = O.draft(tiny["DW"], CFG, tiny["cache"], tiny["hid"], tiny["ref_t0"], tiny["length"], K,
                  head_mode=mode, k_c=max(k_c, 1))
    assert got == ref
    assert eng.device_error() == 0


@pytest.mark.parametrize("mode,k_c", [("clustered", 1), ("clustered", 3), ("full", 1)])
def test_drafter_trace_matches_oracle(tiny, mode, k_c):
    """The drafter's intermediate values of every sub-step (head input, next hidden, centroid
    and token scores) against the oracle at the fp32 tolerance, and its integer choices from its
    own scores; at fp32 no sub-step may need the near-tie allowance."""
    CFG = tiny["cfg"]
    restore(tiny["eng"], tiny["snap"])
    flips = drafter_trace_check(tiny["eng"], CFG, tiny["DW"], tiny["cache"], tiny["hid"],
                                tiny["ref_t0"], tiny["length"], CFG.draft_k, mode, k_c, TOL)
    assert flips == []


def _spec_steps(eng, cur, steps, K, inj):
    """`steps` speculative steps from the current token tensor cur [1] (updated in place);
    returns the emitted tokens."""
    dev = eng.kv_k.device
    drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
    T = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    out = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    n_emit = torch.empty(1, dtype=torch.int32, device=dev)
    toks = []
    for _ in range(steps):
        eng.draft(cur, drafts, inject=inj, verify_tokens=T)
        eng.verify(T)
        eng.accept(T, out_tokens=out, n_emit=n_emit, next_tok=cur, commit=True)
        e = int(n_emit.item())
        toks.extend(out[0, :e].cpu().tolist())
        eng.set_len_bound([int(eng.len[0].item())])
    return toks


def test_snapshot_restore_continues_bitwise(tiny):
    """Snapshot the step state (KV cache, len, hid, next token) mid-generation, run other steps
    that overwrite the cache past len and move len and hid, restore, and continue: the tokens,
    len and hid equal those of an uninterrupted run bit for bit."""
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    K = CFG.draft_k
    dev = eng.kv_k.device
    restore(eng, tiny["snap"])
    ref = gpu_greedy(eng, tiny["t0"], 64)
    L = tiny["length"]
    gseq = np.full(MAX_CTX, -1, dtype=np.int64)
    gseq[L:L + len(ref)] = ref
    inj = torch.from_numpy(inject_table(gseq, K, 0.6, CFG.inject_seed).reshape(1, -1)).to(dev)
    restore(eng, tiny["snap"])
    cur = torch.tensor([tiny["t0"]], dtype=torch.int32, device=dev)
    a = _spec_steps(eng, cur, 12, K, inj)
    end_len, end_hid = eng.len.clone(), eng.hid.clone()

    restore(eng, tiny["snap"])
    cur = torch.tensor([tiny["t0"]], dtype=torch.int32, device=dev)
    b = _spec_steps(eng, cur, 5, K, inj)
    snap = (eng.kv_k.clone(), eng.kv_v.clone(), eng.len.clone(), eng.hid.clone(), cur.clone())
    other = torch.tensor([7], dtype=torch.int32, device=dev)
    _spec_steps(eng, other, 3, K, None)  # different tokens: the cache past len is overwritten
    assert not torch.equal(eng.len, snap[2])
    eng.kv_k.copy_(snap[0])
    eng.kv_v.copy_(snap[1])
    eng.len.copy_(snap[2])
    eng.hid.copy_(snap[3])
    eng.set_len_bound(snap[2].cpu().tolist())
    cur = snap[4].clone()
    b += _spec_steps(eng, cur, 7, K, inj)
    assert b == a
    assert torch.equal(eng.len, end_len) and torch.equal(eng.hid, end_hid)
    assert eng.device_error() == 0


def test_rollback_poison_is_never_read(tiny):
    """Dead cache slots after each rollback are filled with NaN in every layer; the speculative
    output is unchanged and no NaN is flagged."""
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    K = CFG.draft_k
    dev = eng.kv_k.device
    restore(eng, tiny["snap"])
    ref = gpu_greedy(eng, tiny["t0"], 48 + K + 2)
    L = tiny["length"]
    gseq = np.full(MAX_CTX, -1, dtype=np.int64)
    gseq[L:L + len(ref)] = ref
    inj = torch.from_numpy(inject_table(gseq, K, 0.6, CFG.inject_seed).reshape(1, -1)).to(dev)
    restore(eng, tiny["snap"])
    saved = (eng.kv_k.clone(), eng.kv_v.clone())  # the fixture's cache is shared
    kv_k, kv_v = eng.kv_view()
    cur = torch.tensor([tiny["t0"]], dtype=torch.int32, device=dev)
    toks, length, rejected = [tiny["t0"]], L, 0
    while len(toks) < 48:
        toks += _spec_steps(eng, cur, 1, K, inj)
        new_len = int(eng.len[0].item())
        if new_len < length + K + 1:
            rejected += 1
            kv_k[:, 0, :, new_len:length + K + 1, :] = float("nan")
            kv_v[:, 0, :, :, new_len:length + K + 1] = float("nan")
        length = new_len
    assert rejected > 0
    assert toks[:48] == ref[:48]
    assert eng.device_error() == 0
    eng.kv_k.copy_(saved[0])
    eng.kv_v.copy_(saved[1])


def test_nan_norm_weight_raises_the_nan_bit():
    """A NaN in the final norm weight makes every logit NaN: the step flags SPECDEC_DEVERR_NAN
    (the kernels finish normally; nothing is read or written out of bounds)."""
    class NanNorm:
        def __init__(self, src):
            self.src = src

        def get(self, name, layer, shape):
            t = self.src.get(name, layer, shape)
            if name == "final_norm":
                t[3] = float("nan")
            return t

    eng = build_engine(CFG, 64, weights_override=lambda s: NanNorm(s))
    dev = eng.kv_k.device
    am = torch.empty(1, 2, dtype=torch.int32, device=dev)
    eng.verify(torch.tensor([[5, 9]], dtype=torch.int32, device=dev), argmax=am)
    err = eng.device_error(clear=True)
    assert err & SD.ffi.DEVERR_NAN
    assert eng.device_error() == 0  # cleared
    eng.close()


def test_accept_bit_exact_all_patterns(tiny):
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    K = CFG.draft_k
    dev = eng.kv_k.device
    greedy = tiny["gpu_greedy"] if "gpu_greedy" in tiny else None
    if greedy is None:
        restore(eng, tiny["snap"])
        greedy = gpu_greedy(eng, tiny["t0"], K + 2)
    for pattern in itertools.product([0, 1], repeat=K):
        restore(eng, tiny["snap"])
        T = [tiny["t0"]] + [greedy[j + 1] if pattern[j] else (greedy[j + 1] + 7) % CFG.vocab
                            for j in range(K)]
        Tt = torch.tensor([T], dtype=torch.int32, device=dev)
        am = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
        eng.verify(Tt, argmax=am)
        out = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
        n_emit = torch.empty(1, dtype=torch.int32, device=dev)
        nxt = torch.empty(1, dtype=torch.int32, device=dev)
        eng.accept(Tt, out_tokens=out, n_emit=n_emit, next_tok=nxt, commit=True)
        G = am[0].cpu().tolist()
        m, emit, nx = O.accept(T, G)
        m_expect = next((j for j, bit in enumerate(pattern) if not bit), K)
        assert m == m_expect
        assert int(n_emit.item()) == m + 1
        assert out[0, : m + 1].cpu().tolist() == emit == greedy[1 : m + 2]
        assert all(v == -1 for v in out[0, m + 1:].cpu().tolist())
        assert int(nxt.item()) == nx
        assert int(eng.len[0].item()) == tiny["length"] + m + 1
        # committed hidden = hidden of verify row m (compare against the oracle's row)
        cache = tiny["cache"].copy()
        _, H, _ = O.verify(tiny["W"], CFG, cache, tiny["length"], T)
        assert rel_err(eng.hid[0].cpu().numpy(), H[m]) < TOL


def test_argmax_ties_pick_lowest_id():
    """Duplicate the winning embedding row into a lower id: logits tie exactly and the lower id
    must win on the GPU as in the oracle."""
    prompt = prompt_tokens(CFG)[0][:8]
    W, _ = oracle_model(CFG)
    cache = O.KVCache.empty(CFG, 64)
    lg = None
    for pos, tok in enumerate(prompt):
        lg, _ = O.target_row(W, CFG, cache, int(tok), pos)
    win = O.argmax_first(lg)
    low = 0 if win != 0 else 1
    assert low < win or win == 0

    class Dup:
        def __init__(self, src):
            self.src = src

        def get(self, name, layer, shape):
            t = self.src.get(name, layer, shape)
            if name == "embed":
                t[low] = t[win]
            return t

    eng = build_engine(CFG, 64, weights_override=lambda s: Dup(s))
    t0, _ = gpu_prefill(eng, prompt, want_logits=False)
    W["embed"][low] = W["embed"][win]
    cache = O.KVCache.empty(CFG, 64)
    for pos, tok in enumerate(prompt):
        lg, _ = O.target_row(W, CFG, cache, int(tok), pos)
    assert O.argmax_first(lg) == min(low, win)
    assert t0 == min(low, win)
    eng.close()


@pytest.mark.parametrize("pattern", ["all-zero", "copies-of-three"])
def test_moe_routing_ties_pick_lowest_ids(pattern):
    """Router weights whose logits tie exactly: all rows zero (every logit +-0, so the top-k are
    the lowest ids, 0..3), or row e a copy of row e % 3 (three values, each repeated at ids
    congruent mod 3: the top-k are the lowest ids holding the largest value, with the k-th pick
    decided among equal logits).  The GPU must choose the experts the oracle chooses: the logits of
    every prompt row match."""
    cfg = preset("tiny-moe")
    prompt = prompt_tokens(cfg)[0][:32]

    def tie(r):  # a numpy array (oracle) or a device tensor (weight source)
        r = r.clone() if hasattr(r, "clone") else np.array(r, copy=True)
        if pattern == "all-zero":
            r[:] = 0
        else:
            for e in range(r.shape[0]):
                r[e] = r[e % 3]
        return r

    class Ties:
        def __init__(self, src):
            self.src = src

        def get(self, name, layer, shape):
            t = self.src.get(name, layer, shape)
            return tie(t) if name == "router" else t

    eng = build_engine(cfg, 64, weights_override=lambda s: Ties(s))
    try:
        t0, logits = gpu_prefill(eng, prompt)
        W, _ = oracle_model(cfg)
        for lw in W["layers"]:
            lw["router"] = tie(lw["router"])
        cache = O.KVCache.empty(cfg, 64)
        for pos, tok in enumerate(prompt):
            ref, _ = O.target_row(W, cfg, cache, int(tok), pos)
            assert rel_err(logits[pos], ref) < TOL, f"row {pos}"
        assert eng.device_error() == 0
    finally:
        eng.close()


def test_error_paths(tiny):
    CFG = tiny["cfg"]
    eng = tiny["eng"]
    dev = eng.kv_k.device
    restore(eng, tiny["snap"])
    with pytest.raises(SD.SpecdecError) as e:
        eng.verify(torch.zeros(2, 4, dtype=torch.int32, device=dev))  # B > max_batch
    assert e.value.code == -1
    d = torch.empty(1, CFG.draft_k + 5, dtype=torch.int32, device=dev)
    with pytest.raises(SD.SpecdecError):
        eng.draft(torch.zeros(1, dtype=torch.int32, device=dev), d)  # K > max_draft
    d = torch.empty(1, 2, dtype=torch.int32, device=dev)
    with pytest.raises(SD.SpecdecError):
        eng.draft(torch.zeros(1, dtype=torch.int32, device=dev), d, k_c=0)
    # host-side capacity bound
    eng.set_len_bound([MAX_CTX - 2])
    with pytest.raises(SD.SpecdecError) as e:
        eng.verify(torch.zeros(1, 4, dtype=torch.int32, device=dev))
    assert e.value.code == -2
    # a draft's last query position len + K - 1 must be a cache slot
    d = torch.empty(1, 3, dtype=torch.int32, device=dev)
    with pytest.raises(SD.SpecdecError) as e:
        eng.draft(torch.zeros(1, dtype=torch.int32, device=dev), d)
    assert e.value.code == -2
    eng.set_len_bound([MAX_CTX - 3])
    eng.len.fill_(MAX_CTX - 3)
    eng.draft(torch.zeros(1, dtype=torch.int32, device=dev), d)  # positions up to MAX_CTX - 1
    assert eng.device_error(clear=True) == 0
    # device-side guard: len beyond the bound known to the host -> error bit, no write past max_ctx
    before_k = eng.kv_k.clone()
    eng.len.fill_(MAX_CTX - 2)
    eng.set_len_bound([0])
    eng.verify(torch.zeros(1, 4, dtype=torch.int32, device=dev))
    err = eng.device_error(clear=True)
    assert err & SD.ffi.DEVERR_CAPACITY
    kv = eng.kv_view()[0]
    # rows MAX_CTX-2 and MAX_CTX-1 may be written, nothing else changed in the last layer's cache
    changed = (kv != before_k.view(kv.shape)).any(dim=-1)
    assert not changed[..., : MAX_CTX - 2].any()
    # out-of-range token ids raise the token bit and read row 0 instead
    restore(eng, tiny["snap"])
    eng.verify(torch.tensor([[CFG.vocab + 5]], dtype=torch.int32, device=dev))
    assert eng.device_error(clear=True) & SD.ffi.DEVERR_TOKEN
    restore(eng, tiny["snap"])


@pytest.mark.parametrize("name", ["tiny", "tiny-moe"])
def test_batch_of_two_sequences(name):
    """Two sequences in one call: each decodes exactly as it does alone (the path is
    batch-invariant), and the batched speculative loop, with the draft writing the verify rows,
    reproduces the batched greedy output."""
    cfg = preset(name, batch=2)
    n, K = 40, cfg.draft_k
    prompts = prompt_tokens(cfg)
    singles = []
    for b in range(2):
        e1 = build_engine(cfg.replace(batch=1), MAX_CTX)
        t0 = gpu_prefill_batch(e1, prompts[b:b + 1])
        singles.append(gpu_greedy_batch(e1, t0, n)[0])
        e1.close()
    eng = build_engine(cfg, MAX_CTX, max_batch=2)
    t0s = gpu_prefill_batch(eng, prompts)
    snap = snapshot(eng)
    g2 = gpu_greedy_batch(eng, t0s, n + K + 2)
    assert [g[:n] for g in g2] == singles
    L = prompts.shape[1]
    tabs = []
    for b in range(2):
        gseq = np.full(MAX_CTX, -1, dtype=np.int64)
        gseq[L:L + len(g2[b])] = g2[b]
        tabs.append(inject_table(gseq, K, 0.6, cfg.inject_seed, b=b))
    restore(eng, snap)
    toks, emitted = gpu_spec_batch(eng, t0s, n, K, np.stack(tabs))
    assert toks == [g[:n] for g in g2]
    assert all(1 <= e <= K + 1 for step in emitted for e in step)
    assert eng.device_error() == 0
    eng.close()
