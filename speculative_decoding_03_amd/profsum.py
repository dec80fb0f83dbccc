"""Summaries of rocprofv3 output: per-kernel time statistics and HBM traffic per dispatch.

HBM traffic comes from two counter passes (FETCH_SIZE, then WRITE_SIZE, both in KiB per
dispatch).  Each is scaled by what the same counter reads for a plain device copy of known size
(``copy`` below), so that the figure is in real bytes.

  python -m speculative_decoding_03_amd.profsum copy [--mib 1024] [--reps 4]
      runs the plain copy that calibrates the counters (profile it under rocprofv3 --pmc)
  python -m speculative_decoding_03_amd.profsum stats DIR --cmd CMD [--match S --last N] -o OUT
      kernel time table from DIR/*kernel_stats.csv (+ the last N dispatches of kernels whose
      name contains S, from DIR/*kernel_trace.csv)
  python -m speculative_decoding_03_amd.profsum step DIR --index I --cmd CMD -o OUT
      kernels of the I-th target pass (embed to accept) of DIR/*kernel_trace.csv
  python -m speculative_decoding_03_amd.profsum traffic --fetch D --write D --copy-fetch D
      --copy-write D --match S --last N --algorithmic BYTES --src FILE --cmd CMD -o OUT
      per-dispatch HBM bytes of the matching kernel, written as JSON
  python -m speculative_decoding_03_amd.profsum prefill DIR --config NAME --tokens T --cmd CMD
      per-kernel time and TFLOP/s of the last prompt prefill call (embed to commit_rows) of
      DIR/*kernel_trace.csv, with each kernel class's product count from the model's shapes
  python -m speculative_decoding_03_amd.profsum pass --fetch D --write D --copy-fetch D
      --copy-write D [--mfma D --cus N] --index I --algorithmic BYTES --cmd CMD -o OUT
      HBM bytes of every target pass (embed to accept, all kernels) from counter passes taken
      without a kernel filter, against the pass's algorithmic bytes; with --mfma (a pass of
      SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE) also the MFMA busy fraction
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys


def _one(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, f"*{suffix}")))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def short_name(n: str) -> str:
    n = n.replace("void ", "").replace("specdec::", "").replace("(anonymous namespace)::", "")
    n = n.replace("bf16_t", "bf16")
    m = re.match(r"([\w:]+)(<[^()]*>)?", n)
    return (m.group(1) + (m.group(2) or "")) if m else n


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _grid(r) -> int:
    g = r.get("Grid_Size_X", r.get("Grid_Size", "0"))
    return int(float(g))


def trace_rows(d: str):
    """Kernel dispatch rows of a rocprofv3 kernel trace: DIR/*kernel_trace.csv (--output-format
    csv) or the kernels view of DIR/*results.db (the default SQLite output), with the csv
    columns Kernel_Name, Dispatch_Id, Start_Timestamp, End_Timestamp and Grid_Size."""
    csvs = sorted(glob.glob(os.path.join(d, "*kernel_trace.csv")))
    if csvs:
        return _rows(csvs[0])
    import sqlite3
    db = sqlite3.connect(_one(d, "results.db"))
    q = "select name, dispatch_id, start, end, grid_x * grid_y * grid_z from kernels"
    return [{"Kernel_Name": n, "Dispatch_Id": str(i), "Start_Timestamp": str(s),
             "End_Timestamp": str(e), "Grid_Size": str(g)} for n, i, s, e, g in db.execute(q)]


def trace_durations(d: str, match: str, grid: int = 0):
    """Durations (ns) of the dispatches whose kernel name contains `match` (and whose grid has
    `grid` work-items, when given), in dispatch order."""
    rows = [r for r in trace_rows(d) if match in short_name(r["Kernel_Name"])
            and (not grid or _grid(r) == grid)]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def counter_values(d: str, counter: str, match: str | None, grid: int = 0):
    """Per-dispatch value of `counter` for kernels whose short name contains `match` (all
    kernels when None) and whose grid has `grid` work-items (when given), in dispatch order,
    with the kernel names."""
    out = []
    for r in _rows(_one(d, "counter_collection.csv")):
        if r.get("Counter_Name") != counter:
            continue
        name = short_name(r["Kernel_Name"])
        if match is not None and match not in name:
            continue
        if grid and _grid(r) != grid:
            continue
        out.append((int(r["Dispatch_Id"]), name, float(r["Counter_Value"])))
    out.sort()
    return out


def cmd_copy(a) -> int:
    import torch

    n = a.mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": a.reps}))
    return 0


def cmd_stats(a) -> int:
    rows = _rows(_one(a.dir, "kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics", "", f"command: {a.cmd}", ""]
    lines.append(f"{'kernel':<58} {'calls':>7} {'avg us':>10} {'min us':>9} {'max us':>9} {'time %':>7}")
    for r in rows[: a.top]:
        lines.append(f"{short_name(r['Name'])[:58]:<58} {r['Calls']:>7} "
                     f"{float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>9.2f} "
                     f"{float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    if a.match:
        dur = trace_durations(a.dir, a.match, a.grid)
        sel = dur[-a.last:] if a.last else dur
        if sel:
            lines += ["", f"dispatches of '{a.match}' (grid {a.grid or 'any'}): {len(dur)}; "
                      f"the last {len(sel)}: avg {sum(sel) / len(sel) / 1e3:.2f} us, "
                      f"min {min(sel) / 1e3:.2f} us, max {max(sel) / 1e3:.2f} us"]
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    sys.stdout.write(text)
    return 0


def cmd_step(a) -> int:
    """Kernels of one target pass (embed_kernel through accept_kernel), grouped by kernel and grid,
    with the gaps between consecutive kernels."""
    rows = trace_rows(a.dir)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if "embed_kernel" in r["Kernel_Name"]]
    s = starts[a.index]
    e = next(i for i in range(s, len(rows)) if "accept_kernel" in rows[i]["Kernel_Name"])
    agg, order = {}, []
    gaps = 0
    for i in range(s, e + 1):
        r = rows[i]
        k = (short_name(r["Kernel_Name"]), _grid(r))
        if k not in agg:
            agg[k] = [0, 0]
            order.append(k)
        agg[k][0] += 1
        agg[k][1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if i > s:
            gaps += max(0, int(r["Start_Timestamp"]) - int(rows[i - 1]["End_Timestamp"]))
    span = int(rows[e]["End_Timestamp"]) - int(rows[s]["Start_Timestamp"])
    lines = ["# one target pass from a rocprofv3 kernel trace", "", f"command: {a.cmd}", "",
             f"pass {a.index} of {len(starts)}: span {span / 1e3:.1f} us, {e - s + 1} kernels, "
             f"gaps between kernels {gaps / 1e3:.1f} us", "",
             f"{'kernel':<40} {'grid':>9} {'calls':>6} {'total us':>10} {'avg us':>8}"]
    for k in sorted(order, key=lambda k: -agg[k][1]):
        n, t = agg[k]
        lines.append(f"{k[0][:40]:<40} {k[1]:>9} {n:>6} {t / 1e3:>10.1f} {t / n / 1e3:>8.2f}")
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    sys.stdout.write(text)
    return 0


def cmd_prefill(a) -> int:
    """Kernels of the last prefill call (embed_kernel through commit_rows_kernel), with the
    multiply-add count of each prompt-GEMM class and of the causal chunk attention (the chunk of T
    rows starts after the configuration's context)."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import preset
    cfg = preset(a.config)
    T, L = a.tokens, cfg.n_layers
    d, qd, kvd, F = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    keys = sum(cfg.ctx + r + 1 for r in range(T))
    flops = {  # by kernel name prefix and epilogue
        "mm_kernel<1,": ("q/k/v + RoPE + KV append", 2.0 * T * L * d * (qd + 2 * kvd)),
        "mm_kernel<0,": ("o + down (residual add)", 2.0 * T * L * (qd * d + F * d)),
        "mm_kernel<2,": ("gate/up + SiLU product", 2.0 * T * L * d * 2 * F),
        "mm_kernel<3,": ("tied LM head + argmax", 2.0 * T * d * cfg.vocab),
        "attn_prompt_kernel": ("causal prompt attention", 4.0 * L * cfg.n_q_heads * cfg.head_dim * keys),
        "attn_kernel": ("causal chunk attention", 4.0 * L * cfg.n_q_heads * cfg.head_dim * keys),
    }
    rows = trace_rows(a.dir)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    s = [i for i, r in enumerate(rows) if "embed_kernel" in r["Kernel_Name"]][-1]
    e = next(i for i in range(s, len(rows)) if "commit_rows_kernel" in rows[i]["Kernel_Name"])
    agg, order = {}, []
    for i in range(s, e + 1):
        r = rows[i]
        k = short_name(r["Kernel_Name"]).replace(" ", "")
        if k not in agg:
            agg[k] = [0, 0]
            order.append(k)
        agg[k][0] += 1
        agg[k][1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    span = (int(rows[e]["End_Timestamp"]) - int(rows[s]["Start_Timestamp"])) * 1e-9
    total = sum(f for k, (_, f) in flops.items() if k != "attn_kernel")  # attention once
    peak = a.peak_tflops
    lines = [f"## {a.config}: {T} tokens at position {cfg.ctx}", "", f"command: {a.cmd}", "",
             f"last call: span {span * 1e6:.1f} us, {total / 1e12:.2f} TFLOP of GEMM and attention "
             f"work -> {total / span / 1e12:.1f} TFLOP/s ({100 * total / span / 1e12 / peak:.1f}% "
             f"of the {peak / 1000:g} PFLOP/s dense bf16 MFMA peak)", "", "```",
             f"{'kernel':<36} {'calls':>6} {'total us':>10} {'avg us':>9} {'TFLOP/s':>8}  what"]
    for k in sorted(order, key=lambda k: -agg[k][1]):
        n, t = agg[k]
        what, f = next(((w, f) for pre, (w, f) in flops.items() if pre in k), ("", 0.0))
        tf = f"{f / (t * 1e-9) / 1e12:8.1f}" if f else f"{'-':>8}"
        lines.append(f"{k[:36]:<36} {n:>6} {t / 1e3:>10.1f} {t / n / 1e3:>9.2f} {tf}  {what}")
    lines.append("```")
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    sys.stdout.write(text)
    return 0


def _copy_factor(d: str, counter: str, known: float):
    vals = counter_values(d, counter, None)
    if not vals:
        raise SystemExit(f"no {counter} values under {d}")
    # the calibration copy is the dispatch with the largest count
    big = max(v for _, _, v in vals)
    hits = [v for _, _, v in vals if v >= 0.5 * big]
    kib = sum(hits) / len(hits)
    name = [n for _, n, v in vals if v == big][0]
    return known / (kib * 1024.0), kib, name


def cmd_traffic(a) -> int:
    known = a.copy_mib * (1 << 20)
    ff, fkib, fname = _copy_factor(a.copy_fetch, "FETCH_SIZE", known)
    fw, wkib, wname = _copy_factor(a.copy_write, "WRITE_SIZE", known)
    fv = [v for _, _, v in counter_values(a.fetch, "FETCH_SIZE", a.match, a.grid)]
    wv = [v for _, _, v in counter_values(a.write, "WRITE_SIZE", a.match, a.grid)]
    if a.last:
        fv, wv = fv[-a.last:], wv[-a.last:]
    if not fv or not wv:
        raise SystemExit(f"no counter values for '{a.match}'")
    fetch = sum(fv) / len(fv) * 1024.0 * ff
    write = sum(wv) / len(wv) * 1024.0 * fw
    res = {
        "kernel": a.match,
        "grid_work_items": a.grid or None,
        "command": a.cmd,
        "kernel_src": a.src,
        "kernel_src_sha": hashlib.sha256(open(a.src, "rb").read()).hexdigest()[:16],
        "dispatches": {"fetch": len(fv), "write": len(wv)},
        "fetch_kib_per_dispatch_raw": round(sum(fv) / len(fv), 2),
        "write_kib_per_dispatch_raw": round(sum(wv) / len(wv), 2),
        "copy_calibration": {"bytes": known, "kernel": fname, "fetch_kib": round(fkib, 1),
                             "write_kib": round(wkib, 1), "fetch_scale": round(ff, 5),
                             "write_scale": round(fw, 5)},
        "hbm_fetch_bytes_per_dispatch": round(fetch),
        "hbm_write_bytes_per_dispatch": round(write),
        "hbm_bytes_per_dispatch": round(fetch + write),
        "algorithmic_bytes_per_dispatch": a.algorithmic,
        "traffic_over_algorithmic": round((fetch + write) / a.algorithmic, 4) if a.algorithmic else None,
    }
    text = json.dumps(res, indent=1)
    if a.out:
        open(a.out, "w").write(text + "\n")
    print(text)
    return 0


def _passes(vals):
    """Split (dispatch id, name, value) triples, in dispatch order, into target passes: an
    embed_kernel dispatch through the next accept_kernel dispatch."""
    out, cur = [], None
    for t in vals:
        if "embed_kernel" in t[1]:
            cur = [t]
        elif cur is not None:
            cur.append(t)
            if "accept_kernel" in t[1]:
                out.append(cur)
                cur = None
    return out


def cmd_pass(a) -> int:
    known = a.copy_mib * (1 << 20)
    ff, fkib, _ = _copy_factor(a.copy_fetch, "FETCH_SIZE", known)
    fw, wkib, _ = _copy_factor(a.copy_write, "WRITE_SIZE", known)
    fp = _passes(counter_values(a.fetch, "FETCH_SIZE", None))
    wp = _passes(counter_values(a.write, "WRITE_SIZE", None))
    n = min(len(fp), len(wp))
    lines = ["# HBM traffic of whole target passes (rocprofv3 counters, all kernels)", "",
             f"command: {a.cmd}", "",
             f"counters scaled by a plain {a.copy_mib} MiB device copy: FETCH_SIZE x {ff:.5f}, "
             f"WRITE_SIZE x {fw:.5f}", "",
             f"{'pass':>5} {'kernels':>8} {'fetch GB':>10} {'write GB':>10} {'total GB':>10}"]
    tot = []
    for i in range(n):
        f = sum(v for _, _, v in fp[i]) * 1024.0 * ff
        w = sum(v for _, _, v in wp[i]) * 1024.0 * fw
        tot.append((f, w))
        lines.append(f"{i:>5} {len(fp[i]):>8} {f / 1e9:>10.3f} {w / 1e9:>10.3f} {(f + w) / 1e9:>10.3f}")
    f, w = tot[a.index]
    lines += ["", f"pass {a.index}: {(f + w) / 1e9:.3f} GB measured against {a.algorithmic / 1e9:.3f} GB "
              f"algorithmic = {(f + w) / a.algorithmic:.4f}x"]
    if a.mfma:
        # SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs; the capacity of a dispatch is its
        # duration x clock x SIMDs (durations under counter collection run long, so this is a
        # lower bound of the busy fraction)
        rows = [r for r in _rows(_one(a.mfma, "counter_collection.csv"))
                if r.get("Counter_Name") == "SQ_VALU_MFMA_BUSY_CYCLES"]
        trip = sorted((int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]),
                       (float(r["Counter_Value"]),
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))) for r in rows)
        mp = _passes(trip)
        if mp:
            b = sum(v[0] for _, _, v in mp[a.index])
            t = sum(v[1] for _, _, v in mp[a.index]) * 1e-9
            cap = t * a.clock_ghz * 1e9 * a.cus * 4
            lines += [f"pass {a.index}: MFMA busy {b:.4g} SIMD-cycles over {t * 1e3:.2f} ms of its "
                      f"dispatches x {a.clock_ghz} GHz x {a.cus} CUs x 4 SIMDs = {b / cap:.4f} "
                      f"of the MFMA capacity"]
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    sys.stdout.write(text)
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(prog="profsum")
    sp = p.add_subparsers(dest="what", required=True)
    c = sp.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=4)
    s = sp.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--match")
    s.add_argument("--last", type=int, default=0)
    s.add_argument("--grid", type=int, default=0)
    s.add_argument("--top", type=int, default=24)
    s.add_argument("-o", "--out")
    st = sp.add_parser("step")
    st.add_argument("dir")
    st.add_argument("--index", type=int, default=-1)
    st.add_argument("--cmd", required=True)
    st.add_argument("-o", "--out")
    t = sp.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--match", required=True)
    t.add_argument("--last", type=int, default=0)
    t.add_argument("--grid", type=int, default=0)
    t.add_argument("--algorithmic", type=float, default=0.0)
    t.add_argument("--src", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("-o", "--out")
    pf = sp.add_parser("prefill")
    pf.add_argument("dir")
    pf.add_argument("--config", required=True)
    pf.add_argument("--tokens", type=int, default=512)
    pf.add_argument("--peak-tflops", type=float, default=2500.0)
    pf.add_argument("--cmd", required=True)
    pf.add_argument("-o", "--out")
    ps = sp.add_parser("pass")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        ps.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    ps.add_argument("--copy-mib", type=int, default=1024)
    ps.add_argument("--mfma")
    ps.add_argument("--cus", type=int, default=256)
    ps.add_argument("--clock-ghz", type=float, default=2.4)
    ps.add_argument("--index", type=int, default=-1)
    ps.add_argument("--algorithmic", type=float, required=True)
    ps.add_argument("--cmd", required=True)
    ps.add_argument("-o", "--out")
    a = p.parse_args(argv)
    return {"copy": cmd_copy, "stats": cmd_stats, "step": cmd_step, "traffic": cmd_traffic,
            "pass": cmd_pass, "prefill": cmd_prefill}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
