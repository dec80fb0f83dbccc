"""The allocation-free context (specdec_create_static: the workspace is the library's own fixed
array) against the ordinary one (a caller workspace), through the C ABI: the same weights and
inputs give the same outputs bit for bit on two verify calls in a row, the second with fewer
rows, and on a draft; a configuration whose workspace exceeds the array is refused."""

import ctypes as C

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_03_amd as SD  # noqa: E402
from speculative_decoding_03_amd import _ffi as F  # noqa: E402
from speculative_decoding_03_amd import engine as E  # noqa: E402
from workloads import device as WD  # noqa: E402
from workloads import preset, prompt_tokens  # noqa: E402


def test_static_workspace_context_matches_caller_workspace():
    cfg = preset("tiny")
    perm, cent = WD.clusters(cfg)
    model = E.DeviceModel(E.Shape.of(cfg), WD.HostSource(cfg), perm, cent)
    ref = E.Engine(model, max_batch=1, max_draft=3, max_rows=16, max_ctx=128)
    sta = E.Engine(model, max_batch=1, max_draft=3, max_rows=16, max_ctx=128, static_workspace=True)
    assert sta._ws is None and ref.ws_bytes <= F.STATIC_WORKSPACE_BYTES
    dev = ref.kv_k.device
    prompt = prompt_tokens(cfg)[0]
    outs = {}
    for name, eng in (("ref", ref), ("static", sta)):
        got = []
        for rows in (prompt[:16], prompt[16:24]):  # two calls, the second with fewer rows
            toks = torch.tensor(rows, dtype=torch.int32, device=dev).view(1, -1)
            lg = torch.empty(1, len(rows), cfg.vocab, dtype=torch.float32, device=dev)
            am = torch.empty(1, len(rows), dtype=torch.int32, device=dev)
            eng.verify(toks, logits=lg, argmax=am)
            eng.kv_commit(torch.tensor([len(rows)], dtype=torch.int32, device=dev))
            got.append((lg.cpu().numpy(), am.cpu().numpy()))
        eng.set_len_bound([24])
        drafts = torch.empty(1, 3, dtype=torch.int32, device=dev)
        eng.draft(torch.tensor([int(got[-1][1][0, -1])], dtype=torch.int32, device=dev), drafts)
        got.append((drafts.cpu().numpy(),))
        got.append((eng.hid.cpu().numpy(), eng.len.cpu().numpy()))
        assert eng.device_error() == 0
        outs[name] = got
    for a, b in zip(outs["ref"], outs["static"]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    sta.close()
    ref.close()


def test_static_workspace_refuses_a_workspace_beyond_the_array():
    lib = F.load()
    c = F.Config()
    for k, v in dict(n_layers=64, d_model=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
                     ffn_dim=25600, vocab=262144, n_experts=0, top_k=0, expert_ffn=0, shared_ffn=0,
                     d_layers=4, d_dim=256, d_ffn=1024, n_centroids=2048, kv_src_layer=-1,
                     dtype=F.BF16, max_batch=8, max_draft=3, max_rows=8, max_ctx=9216).items():
        setattr(c, k, v)
    c.rms_eps, c.rope_theta = 1e-6, 10000.0
    assert lib.specdec_workspace_bytes(C.byref(c)) > F.STATIC_WORKSPACE_BYTES
    w = F.Weights()
    ctx = C.c_void_p()
    one = C.c_void_p(256)
    rc = lib.specdec_create_static(C.byref(c), C.byref(w), one, one, one, one, None, C.byref(ctx))
    assert rc == F.E_CAPACITY and not ctx.value
