"""GPU parity of the bf16 path at real widths, through the C ABI.

Depth-truncated E2B-shaped (2 layers), E4B-shaped (1 layer; K=4, so a verify call has five
rows and its projections take the row-major activation path), 31B-class (1 layer) and 26B-class
mixture-of-experts (1 layer: 128 experts, top-8, shared FFN) targets keep the full width and
the full 262144-entry vocabulary, each at its workload's committed context (2048, 4096, 8192,
4096 positions: 16 to 64 attention chunks, so the chunk combine runs its main loop), plus an
E2B-shaped case at 700 positions whose drafter keys end inside a chunk.  The 31B, E2B and
mixture-of-experts shapes run again with every weight matrix (embedding, table and centroids
included) in 4-bit blocks; the oracle takes the blocks' exact weights.  Norm weights are
jittered so a dropped norm weight shows.  The oracle computes the hidden rows exactly and the
logits over the whole vocabulary (the embedding is the seeded input generator's, made on the
device bit-identically to the host generator).  Tolerances: max relative error 2e-2 on logits,
hidden states and the drafter's intermediate values; tokens must match wherever the oracle's
top-2 margin exceeds 0.05.  The expert choice of a mixture-of-experts layer is an integer decided
from bf16-input router logits: a row whose oracle gap between the 8th and 9th router logit is
below 0.01 (several times the logits' rounding error) has more than one correct result and is
not compared."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import ctypes as C  # noqa: E402

import oracle as O  # noqa: E402
import speculative_decoding_03_amd as SD  # noqa: E402
from gpu_util import (build_engine, drafter_trace_check, gpu_greedy, gpu_spec,  # noqa: E402
                      gpu_greedy_margins, gpu_spec_tree, host_embedding, oracle_logits_full,
                      rel_err, restore, snapshot)
from workloads import device as WD  # noqa: E402
from workloads import inject_table, truncated  # noqa: E402
from workloads import synth as S  # noqa: E402

TOL = 2e-2
MARGIN = 0.05

CASES = {
    "e2b-L2": truncated("e2b", 2, norm_jitter=0.1, d_layers=2),
    "e2b-L1-ctx700": truncated("e2b", 1, ctx=700, norm_jitter=0.1, d_layers=2),
    "e4b-L1": truncated("e4b", 1, norm_jitter=0.1, d_layers=2),
    "31b-L1": truncated("31b", 1, norm_jitter=0.1, d_layers=2),
    "moe-L1": truncated("moe", 1, norm_jitter=0.1, d_layers=2),
    # every weight matrix in 4-bit blocks (one fp16 step per 32 weights)
    "31b-L1-q4": truncated("31b", 1, norm_jitter=0.1, d_layers=2, weight_format="q4"),
    "e2b-L2-q4": truncated("e2b", 2, norm_jitter=0.1, d_layers=2, weight_format="q4"),
    "moe-L1-q4": truncated("moe", 1, norm_jitter=0.1, d_layers=2, weight_format="q4"),
}
ROUTE_MARGIN = 0.01


def oracle_state(cfg, max_ctx):
    W = O.as_f64({"final_norm": S.norm_weight(cfg, "final_norm", 0, cfg.d_model),
                  "layers": [S.target_layer_weights(cfg, l) for l in range(cfg.n_layers)]})
    k, v = S.kv_init(cfg)
    cache = O.KVCache.from_synthetic(cfg, k[:, 0].astype(np.float64), v[:, 0].astype(np.float64),
                                     max_ctx)
    hid, t0 = S.state_init(cfg)
    return W, cache, hid[0].astype(np.float64), int(t0[0])


def oracle_rows(W, cfg, cache, tokens, length, margins=None):
    """Hidden rows of a verify pass (exact), without the LM head.  `margins`, when given,
    receives each row's smallest routing margin over the layers (inf for a dense model)."""
    H = []
    for i, tok in enumerate(tokens):
        x = O.as_f64(S.gen_rows(cfg, "embed", 0, cfg.d_model, int(tok), 1))[0]
        tr = []
        for l, lw in enumerate(W["layers"]):
            x = O.decoder_layer_row(lw, cfg, cache.K[l], cache.V[l], x, length + i, trace=tr)
        H.append(x)
        if margins is not None:
            margins.append(min(tr, default=np.inf))
    return H


def embed_host(case):
    if "E32" not in case:
        case["E32"] = host_embedding(case["cfg"])
    return case["E32"]


def oracle_full_logits(case, hs):
    return oracle_logits_full(case["cfg"], case["W"], embed_host(case), hs)


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    cfg = CASES[request.param]
    max_ctx = (cfg.ctx + 96 + 7) // 8 * 8
    eng = build_engine(cfg, max_ctx)
    WD.fill_kv(eng, cfg)
    t0 = WD.start_state(eng, cfg)
    W, cache, hid, rt0 = oracle_state(cfg, max_ctx)
    assert int(t0.item()) == rt0
    yield dict(cfg=cfg, eng=eng, W=W, cache=cache, hid=hid, t0=rt0, max_ctx=max_ctx,
               snap=snapshot(eng))
    eng.close()


def test_device_fill_matches_host_generator(case):
    cfg, eng = case["cfg"], case["eng"]
    kv = eng.kv_view()[0]
    for l in range(cfg.n_layers):
        for g in (0, cfg.n_kv_heads - 1):
            ref = S.kv_rows(cfg, "k", l, 0, g, 0, cfg.ctx)
            got = kv[l, 0, g, : cfg.ctx].float().cpu().numpy()
            assert np.array_equal(got, ref)
    src = WD.DeviceSource(cfg)
    ref = S.gen_tensor(cfg, "wo", 0, (cfg.d_model, cfg.q_dim))
    if cfg.weight_format == "q4":
        codes, steps = src.get_q4("wo", 0, (cfg.d_model, cfg.q_dim))
        assert np.array_equal(codes.cpu().numpy(), ref.codes)
        assert np.array_equal(steps.cpu().numpy().view(np.uint16), ref.steps.view(np.uint16))
    else:
        t = src.get("wo", 0, (cfg.d_model, cfg.q_dim)).float().cpu().numpy()
        assert np.array_equal(t, ref)


def test_verify_rows_match_oracle(case):
    cfg, eng = case["cfg"], case["eng"]
    restore(eng, case["snap"])
    K = cfg.draft_k
    rng = np.random.default_rng(11)
    # draft tokens whose rows the oracle routes with a clear margin (always the first draw for a
    # dense model); the current token's row is the same in every draw
    for _ in range(32):
        T = [case["t0"]] + [int(v) for v in rng.integers(0, cfg.vocab, K)]
        margins = []
        H = oracle_rows(case["W"], cfg, case["cache"].copy(), T, cfg.ctx, margins)
        if min(margins[1:]) > ROUTE_MARGIN:
            break
    else:
        pytest.fail("no draw of draft tokens with clear routing margins")
    check_row = [m > ROUTE_MARGIN for m in margins]
    dev = eng.kv_k.device
    Tt = torch.tensor([T], dtype=torch.int32, device=dev)
    logits = torch.empty(1, K + 1, cfg.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    eng.verify(Tt, logits=logits, argmax=am)
    # hidden rows are kept for the commit: commit each row in turn and read hid
    lg = logits[0].cpu().numpy()
    G = am[0].cpu().tolist()
    rows = [i for i in range(K + 1) if check_row[i]]
    ref_all = oracle_full_logits(case, [H[i] for i in rows])
    for i, ref in zip(rows, ref_all):
        restore(eng, case["snap"])
        eng.verify(Tt)
        eng.kv_commit(torch.tensor([i + 1], dtype=torch.int32, device=dev))
        assert rel_err(eng.hid[0].cpu().numpy(), H[i]) < TOL
        # argmax is the lowest-index maximum of the GPU's own logits
        assert G[i] == int(np.argmax(lg[i]))
        # every logit of the vocabulary
        assert rel_err(lg[i], ref) < TOL, f"row {i}: logits"
        # the oracle's full-vocabulary argmax is the GPU's choice unless within the margin
        rb = O.argmax_first(ref)
        if rb != G[i]:
            assert ref[rb] - ref[G[i]] <= MARGIN, f"row {i}: argmax {G[i]} vs oracle {rb}"
    assert eng.device_error() == 0


def test_spec_equals_greedy_and_is_deterministic(case):
    cfg, eng = case["cfg"], case["eng"]
    n, K = 20, cfg.draft_k
    restore(eng, case["snap"])
    g1 = gpu_greedy(eng, case["t0"], n + K + 2)
    restore(eng, case["snap"])
    g2 = gpu_greedy(eng, case["t0"], n + K + 2)
    assert g1 == g2
    gseq = np.full(case["max_ctx"], -1, dtype=np.int64)
    gseq[cfg.ctx:cfg.ctx + len(g1)] = g1
    for p in (0.7, 1.0):
        restore(eng, case["snap"])
        toks, emitted = gpu_spec(eng, case["t0"], n, K, inject_table(gseq, K, p, cfg.inject_seed))
        assert toks == g1[:n]
        if p == 1.0:
            assert all(e == K + 1 for e in emitted)
    assert eng.device_error() == 0


def test_greedy_matches_oracle_teacher_forced(case):
    """The GPU's greedy tokens, scored by the oracle position by position: wherever the oracle's
    margin exceeds 0.05 the GPU token must be the oracle's argmax over the sampled ids."""
    cfg, eng = case["cfg"], case["eng"]
    restore(eng, case["snap"])
    n = 6
    toks = gpu_greedy(eng, case["t0"], n)
    cache = case["cache"].copy()
    Hs = []
    for i in range(n - 1):
        margins = []
        H = oracle_rows(case["W"], cfg, cache, [toks[i]], cfg.ctx + i, margins)
        if margins[0] <= ROUTE_MARGIN:
            break  # a near-tied expert choice: later rows depend on which one was taken
        Hs.append(H[0])
    for i, ref in enumerate(oracle_full_logits(case, Hs)):
        best = O.argmax_first(ref)
        if best != toks[i + 1]:
            assert ref[best] - ref[toks[i + 1]] <= MARGIN


@pytest.mark.parametrize("mode,k_c", [("clustered", 1), ("clustered", 8), ("full", 1)])
def test_drafter_matches_oracle(case, mode, k_c):
    """Every sub-step of a K-token draft: the head input, the next hidden state and the centroid
    scores element by element, the cluster choice and the in-cluster argmax bit-exactly from the
    GPU's own scores (128-token clusters: two argmax units per cluster), the scored tokens against
    the oracle, and the oracle's own choice up to near ties."""
    cfg, eng = case["cfg"], case["eng"]
    restore(eng, case["snap"])
    DW = case.setdefault("DW", O.as_f64(S.drafter_weights(cfg)))
    drafter_trace_check(eng, cfg, DW, case["cache"], case["hid"], case["t0"], cfg.ctx,
                        cfg.draft_k, mode, k_c, TOL, MARGIN)


def test_rollback_leaves_dead_slots_unread(case):
    """After every accept + commit the dead cache slots [len, len_old + K] of every layer are
    filled with NaN: the next draft (keys [0, len)) and verify (which overwrites them first) must
    give the same tokens as without the poison, with no NaN flagged."""
    cfg, eng = case["cfg"], case["eng"]
    n, K = 16, cfg.draft_k
    restore(eng, case["snap"])
    g = gpu_greedy(eng, case["t0"], n + K + 2)
    gseq = np.full(case["max_ctx"], -1, dtype=np.int64)
    gseq[cfg.ctx:cfg.ctx + len(g)] = g
    tab = torch.from_numpy(inject_table(gseq, K, 0.6, cfg.inject_seed).reshape(1, -1)).to(eng.kv_k.device)
    restore(eng, case["snap"])
    saved = (eng.kv_k.clone(), eng.kv_v.clone())  # the fixture's cache is shared
    kv_k, kv_v = eng.kv_view()
    dev = eng.kv_k.device
    cur = torch.tensor([case["t0"]], dtype=torch.int32, device=dev)
    drafts = torch.empty(1, K, dtype=torch.int32, device=dev)
    T = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    out = torch.empty(1, K + 1, dtype=torch.int32, device=dev)
    n_emit = torch.empty(1, dtype=torch.int32, device=dev)
    toks, length, rejected = [case["t0"]], cfg.ctx, 0
    while len(toks) < n:
        eng.draft(cur, drafts, inject=tab, verify_tokens=T)
        eng.verify(T)
        eng.accept(T, out_tokens=out, n_emit=n_emit, next_tok=cur, commit=True)
        e = int(n_emit.item())
        toks.extend(out[0, :e].cpu().tolist())
        lo, hi = length + e, length + K + 1
        if lo < hi:
            rejected += 1
            kv_k[:, 0, :, lo:hi, :] = float("nan")
            kv_v[:, 0, :, :, lo:hi] = float("nan")
        length += e
        eng.set_len_bound([length])
    assert rejected > 0
    assert toks[:n] == g[:n]
    assert eng.device_error() == 0
    eng.kv_k.copy_(saved[0])
    eng.kv_v.copy_(saved[1])


def test_tree_verify_matches_oracle(case):
    """A 2-branch x 3-token tree verified at the workload's width and context: every node's logits
    over the whole vocabulary against the oracle's plain decoding of the node's root path; then
    tree speculation follows greedy decoding up to near ties.  A tree node's key sits in cache
    slot len + node index, not len + depth, so the attention adds the same keys in another order
    than decoding does: the output is exact up to rounding, and a token may differ from the same
    GPU's greedy token only where the greedy step's top-2 margin is within the tolerance."""
    cfg, eng = case["cfg"], case["eng"]
    restore(eng, case["snap"])
    width, depth = 2, 3
    par = O.tree_parents(width, depth)
    g = gpu_greedy(eng, case["t0"], depth + 2)
    restore(eng, case["snap"])
    rng = np.random.default_rng(17)
    # branch 1 holds the greedy tokens for two steps, everything else random
    T = [case["t0"]] + [int(v) for v in rng.integers(0, cfg.vocab, width * depth)]
    T[2], T[4] = g[1], g[2]
    dev = eng.kv_k.device
    Tt = torch.tensor([T], dtype=torch.int32, device=dev)
    lg = torch.empty(1, len(T), cfg.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, len(T), dtype=torch.int32, device=dev)
    eng.verify_tree(par, Tt, logits=lg, argmax=am)
    got = lg[0].cpu().numpy()
    H, check = [], []
    for i in range(len(T)):
        path = O.tree_path(par, i)
        margins = []
        h = oracle_rows(case["W"], cfg, case["cache"].copy(), [T[n] for n in path], cfg.ctx, margins)
        H.append(h[-1])
        check.append(min(margins) > ROUTE_MARGIN)
    rows = [i for i in range(len(T)) if check[i]]
    refs = oracle_full_logits(case, [H[i] for i in rows])
    for i, ref in zip(rows, refs):
        assert rel_err(got[i], ref) < TOL, f"node {i}: logits"
        rb = O.argmax_first(ref)
        if rb != int(am[0, i]):
            assert ref[rb] - ref[int(am[0, i])] <= MARGIN, f"node {i}: argmax"
    assert eng.device_error() == 0
    # tree speculation equals greedy (the same GPU)
    restore(eng, case["snap"])
    n = 16
    ref_g, margins = gpu_greedy_margins(eng, case["t0"], n + depth + 2)
    restore(eng, case["snap"])
    gseq = np.full(case["max_ctx"], -1, dtype=np.int64)
    gseq[cfg.ctx:cfg.ctx + len(ref_g)] = ref_g
    toks, emitted = gpu_spec_tree(eng, case["t0"], n, width, depth,
                                  inject_table(gseq, width * depth, 0.6, cfg.inject_seed))
    for i in range(1, n):
        if toks[i] != ref_g[i]:
            assert margins[i - 1] <= MARGIN, f"token {i} differs at greedy margin {margins[i - 1]:.4f}"
            break
    assert eng.device_error() == 0
