"""Benchmark of the draft-verify-accept step of greedy speculative decoding on one MI355X.

One step = draft K tokens (MTP drafter, clustered head) + verify K+1 rows + fused accept/commit,
on seeded synthetic inputs: random-init bf16 weights of the named shapes (or, with --wformat q4,
every matrix in 4-bit blocks with an fp16 step per 32 weights), a synthetic committed
KV cache of `ctx` positions, and drafts replaced by the target's own greedy token with
probability p (the acceptance mix of the workload).  Inputs are resident in HBM before timing.

Prints one JSON line.  Default workload: the 31B-class dense configuration (64 layers, d 5120,
40/8 heads of 128, FFN 25600, vocab 262144; drafter 4 layers x 256 with 2048 centroids; ctx
8192, K=3, batch 1, p=0.7).  --config e2b | e4b | moe and --batch B run the other workloads.
The default run ends with the same workload on 4-bit weights (a child process, "q4_weights").
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "accepted tokens/s at B=1 (K=3); verify-step ms vs 1-token decode ms; HBM GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
WORKLOAD_TEXT = {
    "31b": "31B-class dense: 64 layers, d 5120, 40 q / 8 kv heads of 128, gated FFN 25600, vocab 262144, bf16 random-init (30.5B params, tied head); drafter 4 layers x 256 over the 5120-d backbone state, 2048 centroids x 128 tokens; ctx 8192, K=3, drafts injected at p=0.7",
    "e2b": "E2B-shaped: 24 layers, d 1536, 8 q / 1 kv heads of 256, gated FFN 6144, vocab 262144, bf16; drafter 4 x 256, 2048 centroids x 128; ctx 2048, K=3, p=0.7",
    "e4b": "E4B-shaped: 34 layers, d 2560, 8 q / 2 kv heads of 256, gated FFN 10240, vocab 262144, bf16; drafter 4 x 256, 2048 centroids; ctx 4096, K=4, p=0.7",
    "31b-tp8": "one GPU's share of the 31B-class model under 8-way tensor parallelism (no collectives): 64 layers, d 5120, 5 q / 1 kv head of 128, gated FFN 3200 (q/k/v 896x5120, o 5120x640, gate/up 6400x5120, down 5120x3200), vocabulary slice 32768 (LM head 32768x5120), bf16; drafter 4 x 256 over the slice, 512 centroids x 64 tokens; ctx 8192, K=3, p=0.7",
    "moe": "26B-class MoE: 30 layers, d 2816, 16 q / 4 kv heads of 176, 128 experts top-8 of FFN 1408 + shared FFN 5632, vocab 262144, bf16 (48.45B params as listed); drafter 4 x 256, 2048 centroids; ctx 4096, K=3, p=0.7",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def wb(cfg) -> float:
    """Bytes per weight: bf16, or the 4-bit block format (half a byte per code plus an fp16 step
    per 32 weights)."""
    return 9 / 16 if cfg.weight_format == "q4" else 2.0


def expert_bytes(cfg) -> float:
    """Bytes of one routed expert's gate, up and down matrices."""
    return 3 * cfg.d_model * cfg.expert_ffn * wb(cfg)


def weight_bytes(cfg, experts_touched: float = 0.0) -> float:
    """Target weight bytes a pass must read: every dense weight once; for a mixture of experts,
    the router and shared FFN of every layer plus the experts the pass's rows were routed to
    (experts_touched, summed over layers)."""
    if not cfg.is_moe:
        return cfg.target_params() * wb(cfg)
    all_experts = cfg.n_layers * cfg.n_experts * expert_bytes(cfg)
    return cfg.target_params() * wb(cfg) - all_experts + experts_touched * expert_bytes(cfg)


def algorithmic_bytes(cfg, B: int, rows: int, keys: float, experts_touched: float = 0.0) -> float:
    """Bytes a verify (rows = K+1) or decode (rows = 1) pass over B sequences must move: the
    target weights once, per sequence and layer the KV of the visible keys and the new rows' KV
    writes, and the embedding rows."""
    kv_read = B * cfg.n_layers * 2 * cfg.n_kv_heads * keys * cfg.head_dim * 2
    kv_write = B * cfg.n_layers * 2 * cfg.n_kv_heads * rows * cfg.head_dim * 2
    return weight_bytes(cfg, experts_touched) + kv_read + kv_write + B * rows * cfg.d_model * 2


def draft_substep_bytes(cfg, B: int, keys: float, k_c: int = 1) -> float:
    D, d, qd = cfg.d_dim, cfg.d_model, cfg.q_dim
    per = D * qd * 2 + 3 * D * cfg.d_ffn
    w = (D * (d + D) + cfg.d_layers * per + d * D + cfg.n_centroids * D) * wb(cfg)
    table = B * (k_c * cfg.cluster_size * D * wb(cfg) + D * wb(cfg))
    kv = B * cfg.d_layers * 2 * cfg.n_kv_heads * keys * cfg.head_dim * 2
    return w + table + kv


def gate_up_bytes(cfg, M: int) -> float:
    """Algorithmic bytes of one gate/up GEMM launch (the dense FFN, or the shared FFN of a
    mixture-of-experts layer): the 2F x d weights once (bf16 or 4-bit blocks), the M bf16 rows of
    x times the norm weight and their per-16-column fp32 sums of squares in, the M bf16
    gated-product rows out."""
    d = cfg.d_model
    F = cfg.shared_ffn if cfg.is_moe else cfg.ffn_dim
    return 2 * F * d * wb(cfg) + M * d * 2 + M * (d // 16) * 4 + M * F * 2


def src_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(name: str, kernel: str, grid: int, launch_bytes: float):
    """HBM traffic of the dominant kernel from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source with the same instantiation, grid and algorithmic bytes;
    else None."""
    p = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        cur = src_sha(os.path.join(ROOT, "speculative_decoding_03_amd", "csrc", "gemm_impl.h"))
        if (d.get("kernel_src_sha") != cur or d.get("kernel") != kernel
                or d.get("grid_work_items") != grid
                or d.get("algorithmic_bytes_per_dispatch") != launch_bytes):
            return None
        return float(d["hbm_bytes_per_dispatch"])
    except Exception:
        return None


def cpu_baseline(cfg, tokens_per_step: float, K: int, B: int) -> dict:
    """The oracle, as it stands, timed on the host's cores on a bounded sample of the same
    workload, for one sequence: the K+1 verify rows through all decoder layers at full width
    against the full synthetic KV (every layer with layer 0's weights: the same shapes, so the
    same work), the tied LM head over a vocabulary slice (scaled to the full vocabulary), and
    the K drafter sub-steps with the clustered head.  B sequences cost B times one."""
    import numpy as np

    import oracle as O
    from workloads import synth as S

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    t_gen = time.perf_counter()
    lw = O.as_f64(S.target_layer_weights(cfg, 0))
    ctx = cfg.ctx
    cap = ctx + K + 2
    Kl = np.zeros((cfg.n_kv_heads, cap, cfg.head_dim))
    Vl = np.zeros_like(Kl)
    for g in range(cfg.n_kv_heads):
        Kl[g, :ctx] = S.kv_rows(cfg, "k", 0, 0, g, 0, ctx)
        Vl[g, :ctx] = S.kv_rows(cfg, "v", 0, 0, g, 0, ctx)
    slice_rows = min(32768, cfg.vocab)
    E_slice = S.gen_rows(cfg, "embed", 0, cfg.d_model, 0, slice_rows).astype(np.float64)
    fnorm = S.norm_weight(cfg, "final_norm", 0, cfg.d_model).astype(np.float64)
    hid, t0 = S.state_init(cfg)
    x0 = hid[0].astype(np.float64)
    DW = O.as_f64(S.drafter_weights(cfg))
    if cfg.is_moe:  # generate the experts the sample routes to outside the timed region
        for i in range(K + 1):
            O.decoder_layer_row(lw, cfg, Kl, Vl, x0, ctx + i)
    gen_s = time.perf_counter() - t_gen

    t = time.perf_counter()
    H = []
    for i in range(K + 1):
        x = x0
        for _ in range(cfg.n_layers):
            x = O.decoder_layer_row(lw, cfg, Kl, Vl, x, ctx + i)
        H.append(x)
    t_layers = time.perf_counter() - t
    t = time.perf_counter()
    for x in H:
        _ = E_slice @ O.rmsnorm(x, fnorm, cfg.rms_eps)
    t_head_slice = time.perf_counter() - t
    t_head = t_head_slice * (cfg.vocab / slice_rows)
    cache = O.KVCache([None] * cfg.n_layers, [None] * cfg.n_layers)
    cache.K[cfg.src_layer] = Kl
    cache.V[cfg.src_layer] = Vl
    t = time.perf_counter()
    O.draft(DW, cfg, cache, x0, int(t0[0]), ctx, K, head_mode="clustered", k_c=1)
    t_draft = time.perf_counter() - t
    step_s = t_layers + t_head + t_draft
    timed = t_layers + t_head_slice + t_draft
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(B * tokens_per_step / (B * step_s), 4),
        "unit": "tokens/s",
        "cores": int(cores),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on {int(cores)} thread{'s' if int(cores) != 1 else ''}, "
                   f"one sequence: the {K + 1} verify "
                   f"rows through all {cfg.n_layers} layers at full width over the {ctx}-position "
                   f"KV, each layer with layer 0's weights ({t_layers:.3g} s); the tied LM head on "
                   f"{slice_rows} of {cfg.vocab} vocabulary rows ({t_head_slice:.3g} s, scaled to "
                   f"{t_head:.3g} s); {K} drafter sub-steps ({t_draft:.3g} s).  {timed:.3g} s timed, "
                   f"one step = {step_s:.3g} s at {tokens_per_step:.2f} tokens/step; input "
                   f"generation {gen_s:.3g} s not timed"),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="31b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--batch", type=int, default=1, help="independent sequences per step")
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--head", default="clustered", choices=["clustered", "full"])
    ap.add_argument("--k-c", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-profile", action="store_true")
    ap.add_argument("--no-p-sweep", dest="p_sweep", action="store_false")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the graph-replay leg (kernel traces then end with the timed steps)")
    ap.add_argument("--sweep-steps", type=int, default=40)
    ap.add_argument("--no-tree", dest="tree", action="store_false", help="skip the tree-draft leg")
    ap.add_argument("--no-adaptive", dest="adaptive", action="store_false",
                    help="skip the adaptive draft-length leg")
    ap.add_argument("--wformat", default="dense", choices=["dense", "q4"],
                    help="weights: bf16, or every matrix in 4-bit blocks with an fp16 step per 32")
    ap.add_argument("--no-q4-leg", dest="q4_leg", action="store_false",
                    help="skip the 4-bit-weight run of the same workload (a child process)")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="skip the streaming-read ceiling measured beside the roofline")
    ap.add_argument("--prefill-tokens", type=int, default=512,
                    help="prompt chunk of the prefill leg (0: none; models without experts)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill leg (for profiling it)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path is built and measured on a single MI355X "
              f"(--gpus {args.gpus} was requested). Multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import speculative_decoding_03_amd as SD
    from speculative_decoding_03_amd import engine as E
    from workloads import device as WD
    from workloads import inject_table, preset

    B = args.batch
    cfg = preset(args.config, batch=B, weight_format=args.wformat)
    if args.p is not None:
        cfg = cfg.replace(p_inject=args.p)
    K, W, N = cfg.draft_k, args.warmup, args.steps
    # steps after the timed region whose gate/up launches are timed one by one (events attached
    # to the dispatches add gaps between kernels, so they stay out of the timed region)
    P = 0 if args.no_kernel_profile else min(N, 8)
    S_all = W + N + P
    head_mode = SD.HEAD_FULL if args.head == "full" else SD.HEAD_CLUSTERED
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    t_setup = time.perf_counter()
    # greedy tokens the injection tables need: every step of the main loop at K+1 tokens, and of
    # the sweep and adaptive legs at up to 7 tokens
    n_greedy = max(S_all * (K + 1), (args.sweep_steps + 2) * (max(K, 6) + 1)) + max(K, 6) + 2
    max_ctx = (cfg.ctx + n_greedy + 64 + 7) // 8 * 8
    log(f"setup {cfg.name}: weights on device ({cfg.target_params() / 1e9:.2f}B target params), B={B}")
    perm, cent = WD.clusters(cfg)
    model = E.DeviceModel(E.Shape.of(cfg), WD.DeviceSource(cfg), perm, cent)
    KA = max(K, 6)  # longest draft the adaptive-length leg may choose
    # verify rows per sequence: a linear step (K + 1, up to KA + 1 in the adaptive leg) or a tree
    # of up to 3 branches (1 + 3K), within the 64 rows of a call
    max_rows = min(64 // B, max(16 // B, KA + 1, 1 + 3 * K))
    PT = args.prefill_tokens if not cfg.is_moe else 0
    max_ctx = max(max_ctx, (cfg.ctx + PT + 7) // 8 * 8)
    eng = E.Engine(model, max_batch=B, max_draft=KA, max_rows=max_rows, max_ctx=max_ctx,
                   max_prefill=PT)
    WD.fill_kv(eng, cfg)
    t0 = WD.start_state(eng, cfg)  # [B] int32
    hid0 = eng.hid.clone()
    torch.cuda.synchronize()
    log(f"setup done in {time.perf_counter() - t_setup:.1f} s")

    def restore():
        eng.hid.copy_(hid0)
        eng.set_len([cfg.ctx] * B)

    def prefill_leg(runs: int = 5) -> dict:
        """One prompt chunk of PT tokens of sequence 0 through the target at position ctx
        (specdec_prefill: compute-bound GEMMs, chunk attention, commit), timed with HIP events
        around the call, inputs resident; the median of `runs` after two warm-up calls."""
        T = PT
        toks = torch.from_numpy(np.random.default_rng(cfg.state_seed + 1)
                                .integers(0, cfg.vocab, T).astype(np.int32)).to(dev)
        am = torch.empty(T, dtype=torch.int32, device=dev)
        ms = []
        for i in range(2 + runs):
            restore()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            eng.prefill(0, toks, argmax=am)
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        assert eng.device_error() == 0, "device error during prefill"
        restore()
        d, qd, kvd = cfg.d_model, cfg.q_dim, cfg.kv_dim
        per_layer = d * (qd + 2 * kvd) + qd * d + 3 * d * cfg.ffn_dim
        gemm = 2.0 * T * (cfg.n_layers * per_layer + cfg.vocab * d)
        keys = sum(cfg.ctx + r + 1 for r in range(T))
        attn = 4.0 * cfg.n_layers * cfg.n_q_heads * cfg.head_dim * keys
        t = float(np.median(ms)) * 1e-3
        return {"tokens": T, "start_position": cfg.ctx, "ms": round(t * 1e3, 3),
                "tokens_per_s": round(T / t, 1),
                "tflops": round((gemm + attn) / t / 1e12, 1),
                "mfma_frac": round((gemm + attn) / t / 1e12 / MFMA_PEAK_TFLOPS, 4),
                "flops": {"gemm": gemm, "attention": attn},
                "what": "specdec_prefill of one sequence: embed, per layer q/k/v + RoPE + KV "
                        "append, causal chunk attention, O, gate/up + SiLU, down (prompt GEMM), "
                        "tied LM head with per-row argmax, commit; bf16 MFMA peak 2.5 PFLOP/s"}

    if args.prefill_only:
        if not PT:
            log("no prefill leg for this configuration")
            return 2
        r = prefill_leg()
        log(f"prefill: {r['tokens']} tokens in {r['ms']} ms, {r['tflops']} TFLOP/s")
        print(json.dumps({"metric": "prefill TFLOP/s", "value": r["tflops"], "unit": "TFLOP/s",
                          "config": {"workload": WORKLOAD_TEXT[args.config]}, "prefill": r}))
        eng.close()
        return 0

    # ---- plain greedy decoding (1-row verify + fused accept/commit): decode-step timing ----
    cur = t0.clone().view(B, 1)
    gbuf = torch.empty(n_greedy, B, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_greedy + 1)]
    torch.cuda.synchronize()
    if cfg.is_moe:
        eng.moe_usage_start()
    ev[0].record()
    for i in range(n_greedy):
        eng.verify(cur)
        eng.accept(cur, out_tokens=gbuf[i].view(B, 1), next_tok=cur, commit=True)
        ev[i + 1].record()
    torch.cuda.synchronize()
    dec_experts = sum(eng.moe_usage_read()) / n_greedy if cfg.is_moe else 0.0
    dec_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(W, n_greedy)]
    g_host = gbuf.cpu().numpy()
    greedy = [[int(t0[b].item())] + g_host[:, b].tolist() for b in range(B)]
    assert eng.device_error() == 0, "device error during greedy decoding"
    log(f"greedy: {n_greedy} decode steps, median {np.median(dec_ms):.3f} ms")

    # ---- speculative loop: draft -> verify -> accept + commit, B sequences per step ----
    def inject_tab(p):
        tabs = []
        for b in range(B):
            gseq = np.full(max_ctx, -1, dtype=np.int64)
            gseq[cfg.ctx:cfg.ctx + len(greedy[b])] = greedy[b]
            tabs.append(inject_table(gseq, K, p, cfg.inject_seed, b=b))
        return torch.from_numpy(np.stack(tabs)).to(dev)

    def spec_run(p, warm, steps, graph=False, prof_steps=0, moe=False):
        """warm + steps (+ prof_steps) speculative steps at injection rate p.  Every step ends
        with one pinned device-to-host copy of its emitted tokens and their count, which the host
        reads one step later (the next step is already enqueued) to learn the committed length;
        the host-side bound on it is then exact up to the one step in flight.  graph=True replays
        one captured step (draft, verify, accept + commit) instead of enqueueing its kernels."""
        restore()
        tab = inject_tab(p)
        S = warm + steps + prof_steps
        cur = t0.clone()
        drafts = torch.empty(B, K, dtype=torch.int32, device=dev)
        T = torch.empty(B, K + 1, dtype=torch.int32, device=dev)  # verify rows, written by the draft
        out_d = torch.full((B, K + 1), -1, dtype=torch.int32, device=dev)
        ne_d = torch.zeros(B, dtype=torch.int32, device=dev)
        out_h = torch.full((S, B, K + 1), -1, dtype=torch.int32).pin_memory()
        ne_h = torch.zeros(S, B, dtype=torch.int32).pin_memory()
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
        e2 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
        done = [torch.cuda.Event() for _ in range(S)]

        def body():
            eng.draft(cur, drafts, head_mode=head_mode, k_c=args.k_c, inject=tab, verify_tokens=T)
            eng.verify(T)
            eng.accept(T, out_tokens=out_d, n_emit=ne_d, next_tok=cur, commit=True)

        g = None
        if graph:
            # captured with the bound at its largest, so that the attention launches cover every
            # chunk a later committed length can reach (the kernels check the device length)
            eng.set_len_bound([max_ctx - (K + 1)] * B)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                body()
            torch.cuda.synchronize()
            restore()
        known = [cfg.ctx] * B

        def enqueue(i):
            e0[i].record()
            if graph:
                g.replay()
                e1[i].record()
            else:
                eng.set_len_bound([n + K + 1 for n in known])  # step i - 1 is still in flight
                eng.draft(cur, drafts, head_mode=head_mode, k_c=args.k_c, inject=tab,
                          verify_tokens=T)
                e1[i].record()
                eng.verify(T)
                eng.accept(T, out_tokens=out_d, n_emit=ne_d, next_tok=cur, commit=True)
            e2[i].record()
            out_h[i].copy_(out_d, non_blocking=True)
            ne_h[i].copy_(ne_d, non_blocking=True)
            done[i].record()

        def read(i):
            done[i].synchronize()
            for b in range(B):
                known[b] += int(ne_h[i, b])

        def run(lo, hi):
            for i in range(lo, hi):
                enqueue(i)
                if i > lo:
                    read(i - 1)
            read(hi - 1)

        run(0, warm)
        torch.cuda.synchronize()
        if moe:
            eng.moe_usage_start()
        t_start = time.perf_counter()
        run(warm, warm + steps)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        experts = sum(eng.moe_usage_read()) / steps if moe else 0.0
        gate = []
        if prof_steps:
            eng.profile_start(SD.ffi.PROF_GATE_UP, cfg.n_layers * prof_steps)
            run(warm + steps, S)
            gate = eng.profile_read()
        assert eng.device_error() == 0, "device error during the speculative loop"
        del g
        ne, ot = ne_h.numpy().copy(), out_h.numpy().copy()
        same = True
        for b in range(B):
            spec = [int(t0[b].item())]
            for i in range(S):
                spec.extend(ot[i, b, : ne[i, b]].tolist())
            same &= spec == greedy[b][: len(spec)]
        timed = range(warm, warm + steps)
        return {"wall": wall, "ne": ne, "same": bool(same), "experts": experts, "gate_ms": gate,
                "emitted": int(ne[warm:warm + steps].sum()),
                "draft_ms": [e0[i].elapsed_time(e1[i]) for i in timed] if not graph else [],
                "ver_ms": [e1[i].elapsed_time(e2[i]) for i in timed] if not graph else [],
                "step_ms": [e0[i].elapsed_time(e2[i]) for i in timed]}

    main = spec_run(cfg.p_inject, W, N, prof_steps=P, moe=cfg.is_moe)
    wall, ne, same = main["wall"], main["ne"], main["same"]
    ver_experts = main["experts"]
    gate_ms = main["gate_ms"]
    draft_ms, ver_ms = main["draft_ms"], main["ver_ms"]
    log(f"speculative loop: {main['emitted'] / wall:.1f} tokens/s, spec == greedy: {same}")
    # graph replay of the whole step, same workload
    try:
        if not args.graph:
            raise RuntimeError("skipped (--no-graph)")
        gr = spec_run(cfg.p_inject, W, N, graph=True)
        log(f"graph replay: {gr['emitted'] / gr['wall']:.1f} tokens/s, spec == greedy: {gr['same']}")
    except Exception as e:  # reported, never the headline
        gr = {"error": f"{type(e).__name__}: {e}"}
        log(f"graph replay failed: {gr['error']}")
    # acceptance mix sweep: p = 0.81 and 0.89 reproduce the pages' tokens-per-pass figures
    sweep = {}
    if args.p_sweep:
        for p in (0.0, 0.6, 0.7, 0.81, 0.89, 1.0):
            r = spec_run(p, 2, args.sweep_steps)
            sweep[str(p)] = {"tokens_per_s": round(r["emitted"] / r["wall"], 2),
                             "tokens_per_step": round(r["emitted"] / (args.sweep_steps * B), 3),
                             "ms_per_step": round(1e3 * r["wall"] / args.sweep_steps, 3),
                             "spec_equals_greedy": r["same"]}
        log("p sweep: " + ", ".join(f"{p}: {v['tokens_per_s']}" for p, v in sweep.items()))

    # draft length chosen per step by the library's policy from the running acceptance, with the
    # costs measured above: one drafter sub-step, a one-row verify, and each further verify row
    adaptive = {}
    if args.adaptive:
        t_sub = float(np.median(main["draft_ms"])) / K
        t_dec = float(np.median(dec_ms))
        t_row = max(0.0, (float(np.median(main["ver_ms"])) - t_dec) / K)
        ktabs = {}

        def adaptive_run(p, steps, warm=2):
            restore()
            for k in range(1, KA + 1):
                tabs = []
                for b in range(B):
                    gseq = np.full(max_ctx, -1, dtype=np.int64)
                    gseq[cfg.ctx:cfg.ctx + len(greedy[b])] = greedy[b]
                    tabs.append(inject_table(gseq, k, p, cfg.inject_seed, b=b))
                ktabs[k] = torch.from_numpy(np.stack(tabs)).to(dev)
            pol = E.KPolicy(1, KA, t_draft_ms=t_sub, t_verify_ms=t_dec, t_row_ms=t_row, decay=0.9)
            cur = t0.clone()
            S = warm + steps
            ne_h = torch.zeros(S, B, dtype=torch.int32).pin_memory()
            out_h = torch.zeros(S, B, KA + 1, dtype=torch.int32).pin_memory()
            done = [torch.cuda.Event() for _ in range(S)]
            toks = [[int(t0[b].item())] for b in range(B)]
            known = [cfg.ctx] * B
            ks, emitted, t_start = [], 0, None
            # one step stays in flight: step i's length is chosen from the steps up to i - 2,
            # and step i - 1's counts are read while step i runs
            def read(i):
                done[i].synchronize()
                ne = ne_h[i].tolist()
                pol.observe(ks_all[i], ne)
                for b in range(B):
                    known[b] += ne[b]
                    toks[b].extend(out_h[i, b, : ne[b]].tolist())
                return sum(ne)
            ks_all = []
            for i in range(S):
                if i == warm:
                    if i > 0:
                        read(i - 1)
                    torch.cuda.synchronize()
                    t_start = time.perf_counter()
                k = pol.choose()
                ks_all.append(k)
                drafts = torch.empty(B, k, dtype=torch.int32, device=dev)
                T = torch.empty(B, k + 1, dtype=torch.int32, device=dev)
                out_d = torch.empty(B, k + 1, dtype=torch.int32, device=dev)
                ne_d = torch.empty(B, dtype=torch.int32, device=dev)
                eng.set_len_bound([n + KA + 1 for n in known])  # one step in flight
                eng.draft(cur, drafts, head_mode=head_mode, k_c=args.k_c, inject=ktabs[k],
                          verify_tokens=T)
                eng.verify(T)
                eng.accept(T, out_tokens=out_d, n_emit=ne_d, next_tok=cur, commit=True)
                ne_h[i].copy_(ne_d, non_blocking=True)
                out_h[i, :, : k + 1].copy_(out_d, non_blocking=True)
                done[i].record()
                if i > 0 and i != warm:
                    e = read(i - 1)
                    if i - 1 >= warm:
                        emitted += e
            emitted += read(S - 1)
            ks = ks_all[warm:]
            torch.cuda.synchronize()
            wall = time.perf_counter() - t_start
            same = all(toks[b] == greedy[b][: len(toks[b])] for b in range(B))
            assert eng.device_error() == 0, "device error in the adaptive-length loop"
            return {"tokens_per_s": round(emitted / wall, 2),
                    "mean_K": round(float(np.mean(ks)), 2),
                    "K_counts": {str(k): ks.count(k) for k in sorted(set(ks))},
                    "final_acceptance_estimate": round(pol.acceptance(), 3),
                    "spec_equals_greedy": bool(same)}

        for p in (0.0, 0.7, 0.89, 1.0):
            r = adaptive_run(p, args.sweep_steps)
            if str(p) in sweep:
                r["fixed_K_tokens_per_s"] = sweep[str(p)]["tokens_per_s"]
            adaptive[str(p)] = r
        log("adaptive K: " + ", ".join(f"{p}: {v['tokens_per_s']} (mean K {v['mean_K']})"
                                       for p, v in adaptive.items()))
    # token trees: width branches of depth K per step, verified in one pass of 1 + width*K rows
    trees = {}
    if args.tree:
        def tree_run(p, width, steps, warm=2):
            restore()
            depth = K
            par = E.tree_parents(width, depth)
            nn = len(par)
            tabs = []
            for b in range(B):
                gseq = np.full(max_ctx, -1, dtype=np.int64)
                gseq[cfg.ctx:cfg.ctx + len(greedy[b])] = greedy[b]
                tabs.append(inject_table(gseq, width * depth, p, cfg.inject_seed, b=b))
            tab = torch.from_numpy(np.stack(tabs)).to(dev)
            S = warm + steps
            cur = t0.clone()
            T = torch.empty(B, nn, dtype=torch.int32, device=dev)
            out_d = torch.empty(B, depth + 1, dtype=torch.int32, device=dev)
            ne_d = torch.empty(B, dtype=torch.int32, device=dev)
            out_h = torch.zeros(S, B, depth + 1, dtype=torch.int32).pin_memory()
            ne_h = torch.zeros(S, B, dtype=torch.int32).pin_memory()
            e0 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
            e1 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
            e2 = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
            done = [torch.cuda.Event() for _ in range(S)]
            known = [cfg.ctx] * B

            def enqueue(i):
                eng.set_len_bound([n + depth + 1 for n in known])  # step i - 1 still in flight
                e0[i].record()
                eng.draft_tree(cur, T, width, depth, head_mode=head_mode, k_c=args.k_c, inject=tab)
                e1[i].record()
                eng.verify_tree(par, T)
                eng.accept_tree(par, T, out_d, n_emit=ne_d, next_tok=cur, commit=True)
                e2[i].record()
                out_h[i].copy_(out_d, non_blocking=True)
                ne_h[i].copy_(ne_d, non_blocking=True)
                done[i].record()

            def read(i):
                done[i].synchronize()
                for b in range(B):
                    known[b] += int(ne_h[i, b])

            for i in range(warm):
                enqueue(i)
                read(i)
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for i in range(warm, S):
                enqueue(i)
                if i > warm:
                    read(i - 1)
            read(S - 1)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t_start
            assert eng.device_error() == 0, "device error in the tree loop"
            ne, ot = ne_h.numpy(), out_h.numpy()
            same = True
            for b in range(B):
                seq = [int(t0[b].item())]
                for i in range(S):
                    seq.extend(ot[i, b, : ne[i, b]].tolist())
                same &= seq == greedy[b][: len(seq)]
            em = int(ne[warm:].sum())
            timed = range(warm, S)
            # steps whose output still follows the greedy reference: a tree node sits in cache slot
            # len + index rather than len + depth, so the attention sums its keys in another order
            # than decoding does, and after a near-tie flip the injected reference tokens no longer
            # apply
            agree, pos = 0, 1
            for i in range(S):
                e = int(ne[i, 0])
                if ot[i, 0, :e].tolist() != greedy[0][pos:pos + e]:
                    break
                pos += e
                agree = i + 1
            step_ms = float(np.median([e0[i].elapsed_time(e2[i]) for i in timed]))
            # expected tokens per step when every node independently holds the reference token
            # with probability p: 1 + sum_j P(some branch agrees through depth j)
            e_tree = 1.0 + sum(1.0 - (1.0 - p ** j) ** width for j in range(1, depth + 1))
            ok = [int(ne[i].sum()) for i in range(warm, min(agree, S))]
            return {"step_ms": round(step_ms, 4),
                    "verify_ms": round(float(np.median([e1[i].elapsed_time(e2[i]) for i in timed])), 4),
                    "draft_ms": round(float(np.median([e0[i].elapsed_time(e1[i]) for i in timed])), 4),
                    "expected_tokens_per_step": round(e_tree, 3),
                    "modelled_tokens_per_s": round(B * e_tree / (step_ms * 1e-3), 2),
                    "measured_tokens_per_step_while_on_reference": round(float(np.mean(ok)) / B, 3) if ok else None,
                    "steps_on_reference": max(0, agree - warm),
                    "wall_tokens_per_s": round(em / wall, 2),
                    "spec_equals_greedy": bool(same)}

        for width in [w for w in (2, 3) if 1 + w * K <= max_rows]:
            for p in (0.7, 0.89):
                r = tree_run(p, width, args.sweep_steps)
                if str(p) in sweep:
                    r["linear_tokens_per_s"] = sweep[str(p)]["tokens_per_s"]
                    r["linear_ms_per_step"] = sweep[str(p)]["ms_per_step"]
                trees[f"width{width}_p{p}"] = r
        log("trees (modelled tokens/s): " + ", ".join(f"{k}: {v['modelled_tokens_per_s']}"
                                                      for k, v in trees.items()))
    emitted = main["emitted"]
    accepted = emitted - N * B
    tok_s = emitted / wall
    med = lambda v: float(np.median(v))  # noqa: E731
    # visible keys of a timed verify: committed length at the step's start + K + 1, averaged
    start_len = cfg.ctx + np.cumsum(np.concatenate([np.zeros((1, B)), ne[:-1]]), axis=0)
    keys_v = float(start_len[W:W + N].mean()) + K + 1
    keys_d = cfg.ctx + n_greedy / 2 + 1
    v_bytes = algorithmic_bytes(cfg, B, K + 1, keys_v, ver_experts)
    d_bytes = algorithmic_bytes(cfg, B, 1, keys_d, dec_experts)
    res = {
        "metric": METRIC,
        "value": round(tok_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": N,
        "warmup": W,
        "ms_per_step": round(1e3 * wall / N, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config] + (
                       "; every weight matrix in 4-bit blocks (fp16 step per 32 weights)"
                       if args.wformat == "q4" else ""),
                   "batch": B, "K": K, "ctx": cfg.ctx, "weights": args.wformat,
                   "p_inject": cfg.p_inject, "head": f"{args.head} k_c={args.k_c}"},
        "verify_ms": round(med(ver_ms), 4),
        "decode_ms": round(med(dec_ms), 4),
        "verify_over_decode": round(med(ver_ms) / med(dec_ms), 4),
        "draft_ms": round(med(draft_ms), 4),
        "p10_p90_ms": {"verify": [round(float(np.percentile(ver_ms, q)), 4) for q in (10, 90)],
                       "decode": [round(float(np.percentile(dec_ms, q)), 4) for q in (10, 90)],
                       "draft": [round(float(np.percentile(draft_ms, q)), 4) for q in (10, 90)]},
        "verify_hbm_gbs": round(v_bytes / (med(ver_ms) * 1e-3) / 1e9, 1),
        "decode_hbm_gbs": round(d_bytes / (med(dec_ms) * 1e-3) / 1e9, 1),
        "verify_hbm_frac": round(v_bytes / (med(ver_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "verify_bytes": round(v_bytes),
        "decode_bytes": round(d_bytes),
        "tokens_per_step": round(emitted / (N * B), 4),
        "accepted_over_proposed": round(accepted / (N * B * K), 4),
        "spec_equals_greedy": bool(same),
        "draft_substep_mb": round(draft_substep_bytes(cfg, B, keys_v) / 1e6, 2),
        "host_readback": "one pinned device-to-host copy of each step's tokens and count, read by "
                         "the host one step later to learn the committed length",
        "graph_replay": gr if "error" in gr else {
            "tokens_per_s": round(gr["emitted"] / gr["wall"], 3),
            "ms_per_step": round(1e3 * gr["wall"] / N, 4),
            "step_ms_median": round(med(gr["step_ms"]), 4),
            "eager_step_ms_median": round(med(main["step_ms"]), 4),
            "spec_equals_greedy": gr["same"]},
    }
    if sweep:
        res["p_sweep"] = sweep
    if trees:
        res["tree_drafts"] = {"shape": f"width branches of depth {K} (1 + width*{K} verify rows)",
                              "tokens_per_s": "modelled: the measured median step time and the "
                                              "expected tokens per step of independent per-node "
                                              "agreement p (output is exact up to rounding, so it "
                                              "leaves the greedy reference at near-ties and the "
                                              "injected reference stops applying)",
                              "by_width_p": trees}
    if adaptive:
        res["adaptive_k"] = {"policy": "library draft-length policy: K in [1, %d] maximising expected "
                                       "tokens per unit time from the decayed acceptance estimate "
                                       "(decay 0.9) and the measured sub-step, decode and per-row "
                                       "costs; per-step host readback" % KA,
                             "by_p": adaptive}
    if cfg.is_moe:
        res["moe"] = {"experts_read_per_verify": round(ver_experts, 1),
                      "experts_read_per_decode": round(dec_experts, 1),
                      "experts_per_layer": cfg.n_experts, "layers": cfg.n_layers}
    if gate_ms:
        launch_ms = float(np.mean(gate_ms))
        M = B * (K + 1)
        lb = gate_up_bytes(cfg, M)
        achieved = lb / (launch_ms * 1e-3) / 1e9
        kw, nu, units, nw, groups = eng.query_launch(0, M)
        q4 = "true" if args.wformat == "q4" else "false"
        kname = f"gemm_kernel<bf16, {1 if M <= 16 else (2 if M <= 32 else 4)}, {nu}, 2, {nw}, false, {q4}>"
        grid = groups * nw * 64
        traffic = load_traffic(f"gemm_gate_up_{args.config}" + (f"_b{B}" if B > 1 else "")
                               + ("_q4" if args.wformat == "q4" else ""), kname, grid, lb)
        what = "shared-FFN gate/up" if cfg.is_moe else "FFN gate/up"
        res["roofline"] = {
            "kernel": f"{kname} ({what} + SiLU product, verify M={M}, grid {grid} work-items, "
                      f"split-K {kw})",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": lb,
            "avg_launch_us": round(launch_ms * 1e3, 2),
            "launches": len(gate_ms),
            "launch_timing": f"HIP events attached to the dispatches; the gate/up launches of {P} "
                             f"speculative steps run after the timed region",
        }
    ceil = {}
    if gate_ms and args.ceiling:
        # a plain streaming read of the dominant launch's bytes beside its roofline: the bandwidth
        # a weight stream of that size reaches on this GPU with no arithmetic at all
        from workloads import device as WD
        ceil = WD.stream_read_ceiling(int(res["roofline"]["algorithmic_bytes_per_launch"]))
    if ceil:
        best = max(ceil.values(), key=lambda r: r["gbs"])
        res["streaming_ceiling"] = {
            "what": "non-temporal 16-byte loads, one contiguous run per wave, 8 in flight per lane, "
                    "over the dominant launch's bytes; by workgroups of 8 waves",
            "by_workgroups": ceil, "best_gbs": best["gbs"],
            "best_frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4),
            "roofline_achieved_over_best": round(res["roofline"]["achieved"] / best["gbs"], 4)}
        log(f"streaming ceiling: {best['gbs']} GB/s ({res['streaming_ceiling']['best_frac_of_peak']} of peak)")
    if PT:
        res["prefill"] = prefill_leg()
        log(f"prefill: {PT} tokens in {res['prefill']['ms']} ms, {res['prefill']['tflops']} TFLOP/s")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores, bounded sample)")
        res["cpu_baseline"] = cpu_baseline(cfg, emitted / (N * B), K, B)
        # the tiny configuration's shapes on one BLAS thread, same step structure (64 committed
        # positions; counter-hash weights, which the sample generators need)
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                tiny = cpu_baseline(preset("tiny", ctx=64, init="hash"), emitted / (N * B), K, 1)
            res["cpu_baseline"]["tiny_one_thread"] = {k: tiny[k] for k in ("value", "unit", "cores",
                                                                             "sample")}
        except ImportError:
            pass
    eng.close()
    del eng, model
    torch.cuda.empty_cache()
    if args.q4_leg and args.wformat == "dense":
        res["q4_weights"] = q4_leg(args)
    print(json.dumps(res), flush=True)
    return 0


def q4_leg(args) -> dict:
    """The same workload with every weight matrix in 4-bit blocks, run as a child process (its
    progress goes to stderr) with the headline's timing and kernel profile, without the sweeps."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--config", args.config, "--batch",
           str(args.batch), "--wformat", "q4", "--steps", str(min(args.steps, 100)), "--warmup",
           str(args.warmup), "--head", args.head, "--k-c", str(args.k_c), "--no-cpu-baseline",
           "--no-p-sweep", "--no-tree", "--no-adaptive", "--no-graph", "--no-q4-leg", "--no-ceiling"]
    if args.p is not None:
        cmd += ["--p", str(args.p)]
    log("4-bit weight leg: " + " ".join(cmd[2:]))
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if r.returncode != 0:
        return {"error": f"exit status {r.returncode}"}
    try:
        d = json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:
        return {"error": f"unreadable output: {e}"}
    keep = ("value", "unit", "steps", "ms_per_step", "verify_ms", "decode_ms", "draft_ms",
            "verify_over_decode", "verify_hbm_gbs", "verify_hbm_frac", "verify_bytes",
            "tokens_per_step", "spec_equals_greedy", "roofline", "prefill")
    out = {k: d[k] for k in keep if k in d}
    out["weights"] = "4-bit blocks: codes plus an fp16 step per 32 weights (0.5625 bytes/weight)"
    return out


if __name__ == "__main__":
    sys.exit(main())
