"""GPU-side workload sources: logical weight tensors, synthetic KV caches and start states.

``HostSource`` uploads the host generator's arrays (small configurations, the tiny fp32 one);
``DeviceSource`` fills hash-initialised tensors directly on the GPU with libsynth.so, which is
bit-identical to the host generator (large configurations).  ``get`` returns a dense tensor;
``get_q4`` the codes and steps of a 4-bit one.  Holds no part of the method.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

from . import synth as S

HERE = os.path.dirname(os.path.abspath(__file__))
SYNTH_LIB = os.path.join(HERE, "libsynth.so")
_synth = None

NORMS = {"attn_norm", "ffn_norm", "final_norm", "norm_h", "norm_e", "d_nf", "d_n1", "d_n2"}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def build_synth(verbose: bool = True) -> str:
    import subprocess
    src = os.path.join(HERE, "csrc", "synth_fill.hip")
    tmp = SYNTH_LIB + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for synth_fill.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, SYNTH_LIB)
    if verbose:
        print(f"built {SYNTH_LIB}")
    return SYNTH_LIB


def synth_lib():
    global _synth
    if _synth is None:
        if not os.path.exists(SYNTH_LIB):
            raise RuntimeError(f"{SYNTH_LIB} is missing: run __graft_entry__.build()")
        lib = C.CDLL(SYNTH_LIB)
        lib.synth_fill_uniform.restype = C.c_int
        lib.synth_fill_uniform.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_uint64, C.c_int64,
                                           C.c_float, C.c_void_p]
        lib.synth_fill_q4.restype = C.c_int
        lib.synth_fill_q4.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_uint64,
                                      C.c_int64, C.c_uint64, C.c_int64, C.c_float, C.c_void_p]
        lib.synth_fill_kv.restype = C.c_int
        lib.synth_fill_kv.argtypes = [C.c_void_p] + [C.c_int] * 8 + [C.c_uint64, C.c_float, C.c_int,
                                                                      C.c_void_p]
        lib.synth_stream_read.restype = C.c_int
        lib.synth_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        _synth = lib
    return _synth


def stream_read_ceiling(nbytes: int, n_wgs=(160, 256, 1600), reps: int = 7) -> dict:
    """Read bandwidth of a plain streaming kernel (non-temporal 16-byte loads, one contiguous run
    per wave, 8 loads in flight per lane) over a buffer of about nbytes, for a few workgroup
    counts (those that give every wave at least 512 loads): the ceiling a weight-streaming GEMM
    of that size can reach.  Median of reps timed
    launches each, a 1 GiB read of another buffer between them (so nothing is served from the
    caches)."""
    dev = torch.device("cuda")
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    flush = torch.ones((1 << 30) // 2, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    lib, st = synth_lib(), _stream()
    out = {}
    for nwg in n_wgs:
        per = (nbytes // 16) // (nwg * 8) // 512 * 512
        if per < 512:  # under one 512-load granule per wave: too many workgroups for the size
            continue
        fper = ((1 << 30) // 16) // (2048 * 8) // 512 * 512
        ms = []
        for _ in range(reps):
            if lib.synth_stream_read(C.c_void_p(flush.data_ptr()), fper, 2048, C.c_void_p(sink.data_ptr()), st):
                raise RuntimeError("synth_stream_read failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if lib.synth_stream_read(C.c_void_p(buf.data_ptr()), per, nwg, C.c_void_p(sink.data_ptr()), st):
                raise RuntimeError("synth_stream_read failed")
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        b = per * 16 * nwg * 8
        out[str(nwg)] = {"bytes": b, "us": round(ms[len(ms) // 2] * 1e3, 2),
                         "gbs": round(b / (ms[len(ms) // 2] * 1e-3) / 1e9, 1)}
    del buf, flush
    return out


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def fill_uniform(t: torch.Tensor, key: int, std: float, start: int = 0) -> torch.Tensor:
    bf16 = 1 if t.dtype == torch.bfloat16 else 0
    rc = synth_lib().synth_fill_uniform(C.c_void_p(t.data_ptr()), t.numel(), bf16, C.c_uint64(key),
                                        start, float(S.hash_scale(std)), _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_uniform failed ({rc})")
    return t


class HostSource:
    """Logical tensors from the host generator, uploaded to the device."""

    def __init__(self, cfg, device="cuda"):
        self.cfg, self.device = cfg, device

    def get(self, name, layer, shape):
        cfg = self.cfg
        if name in NORMS:
            a = S.norm_weight(cfg, name, layer, shape[0])
            return torch.from_numpy(a).to(self.device)
        assert cfg.weight_format == "dense", "4-bit weights come from get_q4"
        a = S.gen_tensor(cfg, name, layer, shape)
        return torch.from_numpy(a).to(device=self.device, dtype=TORCH_DT[cfg.dtype])

    def get_q4(self, name, layer, shape):
        """(codes uint8 [*shape], steps float16 [*shape[:-1], shape[-1] / 32]) on the device."""
        q = S.gen_tensor(self.cfg, name, layer, shape)
        return (torch.from_numpy(q.codes).to(self.device),
                torch.from_numpy(q.steps).to(self.device))


class DeviceSource:
    """Hash-initialised logical tensors generated on the device (bit-identical to HostSource)."""

    def __init__(self, cfg, device="cuda"):
        assert cfg.init == "hash"
        self.cfg, self.device = cfg, device

    def get(self, name, layer, shape):
        cfg = self.cfg
        if name in NORMS:
            return torch.from_numpy(S.norm_weight(cfg, name, layer, shape[0])).to(self.device)
        assert cfg.weight_format == "dense", "4-bit weights come from get_q4"
        t = torch.empty(shape, dtype=TORCH_DT[cfg.dtype], device=self.device)
        return fill_uniform(t, S.stream_key(cfg.seed, S.tensor_id(name, layer)), cfg.weight_std)

    def get_q4(self, name, layer, shape, row_start: int = 0):
        """(codes uint8 [*shape], steps float16 [*shape[:-1], shape[-1] / 32]) on the device; rows
        row_start.. of the tensor when only a slice is wanted."""
        cfg = self.cfg
        K = shape[-1]
        codes = torch.empty(shape, dtype=torch.uint8, device=self.device)
        steps = torch.empty((*shape[:-1], K // 32), dtype=torch.float16, device=self.device)
        tid = S.tensor_id(name, layer)
        rc = synth_lib().synth_fill_q4(
            C.c_void_p(codes.data_ptr()), codes.numel(), C.c_void_p(steps.data_ptr()), steps.numel(),
            C.c_uint64(S.stream_key(cfg.seed, tid)), row_start * K,
            C.c_uint64(S.stream_key(cfg.seed, tid + S.Q4_STEP_TID)), row_start * (K // 32),
            float(S.q4_step_scale(cfg.weight_std)), _stream())
        if rc != 0:
            raise RuntimeError(f"synth_fill_q4 failed ({rc})")
        return codes, steps


def source_for(cfg, device="cuda"):
    return DeviceSource(cfg, device) if cfg.init == "hash" else HostSource(cfg, device)


def clusters(cfg, device="cuda"):
    """(perm, centroids) for the drafter's clustered head.  Centroids are member means of the
    host-generated table, which is bit-identical to the device one; 4-bit weights draw their own
    centroids, returned as (codes, steps) device tensors."""
    perm = S.cluster_perm(cfg)
    if cfg.weight_format == "q4":
        return torch.from_numpy(perm).to(device), source_for(cfg, device).get_q4(
            "centroids", 0, (cfg.n_centroids, cfg.d_dim))
    table = S.gen_tensor(cfg, "table", 0, (cfg.vocab, cfg.d_dim))
    cent = S.centroids_from_table(cfg, table, perm)
    return torch.from_numpy(perm).to(device), torch.from_numpy(cent).to(device)


def fill_kv(engine, cfg) -> None:
    """Synthetic committed KV of cfg.ctx positions for sequences [0, cfg.batch) (std 1); K is
    stored [pos][hd] and V transposed [hd][pos], as the library lays the cache out."""
    bf16 = 1 if cfg.dtype == "bf16" else 0
    s = engine.shape
    for which, buf in (("kv_k", engine.kv_k), ("kv_v", engine.kv_v)):
        key = S.stream_key(cfg.kv_seed, S.tensor_id(which, 0))
        rc = synth_lib().synth_fill_kv(C.c_void_p(buf.data_ptr()), s.n_layers, cfg.batch,
                                       engine.max_batch, s.n_kv_heads, cfg.ctx, engine.max_ctx,
                                       s.head_dim, bf16, C.c_uint64(key), float(S.hash_scale(1.0)),
                                       1 if which == "kv_v" else 0, _stream())
        if rc != 0:
            raise RuntimeError(f"synth_fill_kv failed ({rc})")


def start_state(engine, cfg):
    """Sets len = ctx, hid = synthetic hidden; returns the synthetic current tokens [B] (int32)."""
    hid, t0 = S.state_init(cfg)
    engine.hid[: cfg.batch].copy_(torch.from_numpy(hid))
    engine.set_len([cfg.ctx] * cfg.batch)
    return torch.from_numpy(t0.astype(np.int32)).to(engine.kv_k.device)
