"""GPU parity of batched bf16 verify calls, through the C ABI.

Several independent sequences share one call (the batch of the 26B-class model's batch-4..8
serving case).  Each has its own committed length, so one launch mixes different key counts
and attention chunk counts.  Depth-truncated targets keep the full width and the full
262144-entry vocabulary:
* 31B-class at B=8: 32 verify rows, two 16-row MFMA tiles per projection on the row-major path;
* 26B-class mixture-of-experts at B=4 and B=8: 16 and 32 rows routed over 128 experts, top-8
  (at B=8 the grouped expert GEMMs run two M-tiles);
* a 64-row prefill call at the E2B width (four 16-row M-tiles per projection, 512 query vectors
  per KV head in the attention);
* the 31B-class B=8 case and the prefill call again with every weight matrix in 4-bit blocks.

Every verify row's hidden state and its logits over the whole vocabulary are compared with the
oracle run on that row's own sequence alone, so a row that read another sequence's cache,
length or routing would fail.  Tolerances and the margin rules are those of the
single-sequence bf16 tests."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle as O  # noqa: E402
from gpu_util import (build_engine, gpu_greedy_batch, gpu_spec_batch,  # noqa: E402
                      host_embedding, oracle_logits_full, rel_err)
from workloads import device as WD  # noqa: E402
from workloads import inject_table, truncated  # noqa: E402
from workloads import synth as S  # noqa: E402

TOL = 2e-2
MARGIN = 0.05
ROUTE_MARGIN = 0.01

CASES = {
    "31b-L1-B8": truncated("31b", 1, ctx=530, norm_jitter=0.1, d_layers=2, batch=8),
    "moe-L1-B4": truncated("moe", 1, ctx=530, norm_jitter=0.1, d_layers=2, batch=4),
    "moe-L1-B8": truncated("moe", 1, ctx=530, norm_jitter=0.1, d_layers=2, batch=8),
    "31b-L1-B8-q4": truncated("31b", 1, ctx=530, norm_jitter=0.1, d_layers=2, batch=8,
                              weight_format="q4"),
}
# committed length of each sequence: ctx minus these (different chunk counts in one call)
SHORTEN = [0, 37, 130, 3, 64, 129, 255, 1]


def oracle_rows(W, cfg, cache, tokens, length, margins):
    H = []
    for i, tok in enumerate(tokens):
        x = O.as_f64(S.gen_rows(cfg, "embed", 0, cfg.d_model, int(tok), 1))[0]
        tr = []
        for l, lw in enumerate(W["layers"]):
            x = O.decoder_layer_row(lw, cfg, cache.K[l], cache.V[l], x, length + i, trace=tr)
        H.append(x)
        margins.append(min(tr, default=np.inf))
    return H




@pytest.fixture(scope="module", params=sorted(CASES))
def bcase(request):
    cfg = CASES[request.param]
    B = cfg.batch
    max_ctx = (cfg.ctx + 96 + 7) // 8 * 8
    eng = build_engine(cfg, max_ctx, max_rows=64 // B, max_batch=B)
    WD.fill_kv(eng, cfg)
    t0 = WD.start_state(eng, cfg)
    lens = [cfg.ctx - s for s in SHORTEN[:B]]
    W = O.as_f64({"final_norm": S.norm_weight(cfg, "final_norm", 0, cfg.d_model),
                  "layers": [S.target_layer_weights(cfg, l) for l in range(cfg.n_layers)]})
    k, v = S.kv_init(cfg)
    caches = [O.KVCache.from_synthetic(cfg, k[:, b].astype(np.float64), v[:, b].astype(np.float64),
                                       max_ctx) for b in range(B)]
    hid = eng.hid[:B].clone()
    yield dict(cfg=cfg, eng=eng, W=W, caches=caches, t0=t0.cpu().tolist(), lens=lens, hid=hid,
               max_ctx=max_ctx)
    eng.close()


def reset(c):
    eng = c["eng"]
    eng.set_len(c["lens"])
    eng.hid[: c["cfg"].batch].copy_(c["hid"])


def test_batched_verify_rows_match_oracle(bcase):
    cfg, eng = bcase["cfg"], bcase["eng"]
    B, K = cfg.batch, cfg.draft_k
    rng = np.random.default_rng(23)
    T, H, check = [], [], []
    for b in range(B):
        for _ in range(32):  # draft tokens routed with a clear margin (first draw when dense)
            row = [bcase["t0"][b]] + [int(x) for x in rng.integers(0, cfg.vocab, K)]
            margins = []
            h = oracle_rows(bcase["W"], cfg, bcase["caches"][b].copy(), row, bcase["lens"][b], margins)
            if min(margins[1:]) > ROUTE_MARGIN:
                break
        else:
            pytest.fail(f"sequence {b}: no draw of draft tokens with clear routing margins")
        T.append(row)
        H.append(h)
        check.append([m > ROUTE_MARGIN for m in margins])
    dev = eng.kv_k.device
    Tt = torch.tensor(T, dtype=torch.int32, device=dev)
    logits = torch.empty(B, K + 1, cfg.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    reset(bcase)
    eng.verify(Tt, logits=logits, argmax=am)
    lg = logits.cpu().numpy()
    G = am.cpu().numpy()
    E32 = host_embedding(cfg)
    pairs = [(b, i) for b in range(B) for i in range(K + 1) if check[b][i]]
    refs = dict(zip(pairs, oracle_logits_full(cfg, bcase["W"], E32, [H[b][i] for b, i in pairs])))
    del E32
    for i in range(K + 1):
        # committing i+1 rows leaves each sequence's hidden row i in hid
        reset(bcase)
        eng.verify(Tt)
        eng.kv_commit(torch.full((B,), i + 1, dtype=torch.int32, device=dev))
        got = eng.hid[:B].cpu().numpy()
        assert eng.len[:B].cpu().tolist() == [n + i + 1 for n in bcase["lens"]]
        for b in range(B):
            if not check[b][i]:
                continue
            assert rel_err(got[b], H[b][i]) < TOL, f"sequence {b} row {i}"
            assert G[b, i] == int(np.argmax(lg[b, i]))
            ref = refs[(b, i)]
            assert rel_err(lg[b, i], ref) < TOL, f"sequence {b} row {i}: logits"
            rb = O.argmax_first(ref)
            if rb != G[b, i]:
                assert ref[rb] - ref[G[b, i]] <= MARGIN, f"sequence {b} row {i}: argmax"
    assert eng.device_error() == 0


def test_batched_spec_equals_batched_greedy(bcase):
    cfg, eng = bcase["cfg"], bcase["eng"]
    B, K, n = cfg.batch, cfg.draft_k, 16
    reset(bcase)
    g = gpu_greedy_batch(eng, bcase["t0"], n + K + 2)
    tabs = []
    for b in range(B):
        gseq = np.full(bcase["max_ctx"], -1, dtype=np.int64)
        gseq[bcase["lens"][b]:bcase["lens"][b] + len(g[b])] = g[b]
        tabs.append(inject_table(gseq, K, 0.7, cfg.inject_seed, b=b))
    reset(bcase)
    toks, emitted = gpu_spec_batch(eng, bcase["t0"], n, K, np.stack(tabs))
    assert toks == [s[:n] for s in g]
    assert all(1 <= e <= K + 1 for step in emitted for e in step)
    assert eng.device_error() == 0


def test_gated_units_of_the_batched_call(bcase):
    """A call of 17..32 rows of a dense gate/up projection takes wider units, one per workgroup:
    four gate/up pairs at the 31B width (3200 tiles), two for the narrower shared FFN of the
    mixture-of-experts model (704 tiles), so the verify tests above run both; calls of 16 rows or
    fewer and 4-bit weights keep units of one pair.  The split-K is the same for every call
    size."""
    cfg, eng = bcase["cfg"], bcase["eng"]
    M = cfg.batch * (cfg.draft_k + 1)
    kw, nu, units, nw, groups = eng.query_launch(0, M)
    kw1, nu1, units1, nw1, groups1 = eng.query_launch(0, cfg.batch)
    assert kw == kw1 and nu1 == 2
    tiles = 2 * (cfg.shared_ffn if cfg.is_moe else cfg.ffn_dim) // 16
    wide = 16 < M <= 32 and cfg.weight_format == "dense"
    expect = 2
    if wide and tiles % 8 == 0 and tiles // 8 >= 400:
        expect = 8
    elif wide and tiles % 4 == 0 and tiles // 4 >= 128:
        expect = 4
    assert nu == expect
    assert units * nu == units1 * nu1 and groups == units * kw // nw
    if expect > 2:
        assert nw == max(4, kw)  # one unit per workgroup


@pytest.mark.parametrize("wformat", ["dense", "q4"])
def test_prefill_call_of_64_rows_matches_oracle(wformat):
    """One 64-row verify call (a prefill chunk) at the E2B width after 530 committed positions:
    four 16-row M-tiles per projection and 64 x 8 query vectors per KV head.  Hidden rows at a
    sample of positions, all 64 rows' argmax against the GPU's own logits, and the logits over
    the whole vocabulary of the sampled rows against the oracle; bf16 and 4-bit weights."""
    cfg = truncated("e2b", 1, ctx=530, norm_jitter=0.1, d_layers=2, weight_format=wformat)
    R = 64
    max_ctx = (cfg.ctx + R + 8 + 7) // 8 * 8
    eng = build_engine(cfg, max_ctx, max_rows=R)
    try:
        WD.fill_kv(eng, cfg)
        WD.start_state(eng, cfg)
        W = O.as_f64({"final_norm": S.norm_weight(cfg, "final_norm", 0, cfg.d_model),
                      "layers": [S.target_layer_weights(cfg, l) for l in range(cfg.n_layers)]})
        k, v = S.kv_init(cfg)
        cache = O.KVCache.from_synthetic(cfg, k[:, 0].astype(np.float64), v[:, 0].astype(np.float64),
                                         max_ctx)
        toks = [int(t) for t in np.random.default_rng(41).integers(0, cfg.vocab, R)]
        H = oracle_rows(W, cfg, cache, toks, cfg.ctx, [])
        dev = eng.kv_k.device
        Tt = torch.tensor([toks], dtype=torch.int32, device=dev)
        logits = torch.empty(1, R, cfg.vocab, dtype=torch.float32, device=dev)
        am = torch.empty(1, R, dtype=torch.int32, device=dev)
        eng.verify(Tt, logits=logits, argmax=am)
        lg = logits[0].cpu().numpy()
        G = am[0].cpu().numpy()
        assert all(G[i] == int(np.argmax(lg[i])) for i in range(R))
        sample = [0, 1, 17, 31, 32, 47, 48, 63]
        refs = oracle_logits_full(cfg, W, host_embedding(cfg), [H[i] for i in sample])
        for i, ref in zip(sample, refs):
            eng.set_len([cfg.ctx])
            eng.verify(Tt)
            eng.kv_commit(torch.tensor([i + 1], dtype=torch.int32, device=dev))
            assert rel_err(eng.hid[0].cpu().numpy(), H[i]) < TOL, f"row {i}: hidden"
            assert rel_err(lg[i], ref) < TOL, f"row {i}: logits"
            rb = O.argmax_first(ref)
            if rb != G[i]:
                assert ref[rb] - ref[G[i]] <= MARGIN, f"row {i}: argmax"
        assert eng.device_error() == 0
    finally:
        eng.close()
