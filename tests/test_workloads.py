"""Pins for the seeded input generators (published SplitMix64 outputs, bf16 rounding)."""

import json
import math
import os

import numpy as np

from workloads import (bf16_bits, bf16_from_bits, hash_u64, hash_uniform_f32, inject_draw,
                       inject_threshold, mix64, preset, stream_key)
from workloads.synth import GOLDEN, MASK64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLD, "splitmix64_seed0.json")))
    # The stream with key = initial state 0 yields mix64(0 + (i+1)*gamma) for i = 0, 1, 2.
    z = hash_u64(g["state0"], 0, 3)
    assert [f"{int(v):016x}" for v in z] == g["outputs_hex"]


def test_stream_key_is_first_output_of_state():
    s = (7 << 32) + 12345
    assert stream_key(7, 12345) == int(mix64(np.array([(s + GOLDEN) & MASK64], np.uint64))[0])


def test_bf16_rounding_cases():
    g = json.load(open(os.path.join(GOLD, "bf16_rounding.json")))
    for c in g["cases"]:
        x = np.array([int(c["f32_bits"], 16)], dtype=np.uint32).view(np.float32)
        assert f"{int(bf16_bits(x)[0]):04x}" == c["bf16_bits"]
    # round trip of representable values is exact
    v = bf16_from_bits(np.arange(0, 0x7f80, 97, dtype=np.uint16))
    assert np.array_equal(bf16_from_bits(bf16_bits(v)), v)


def test_hash_uniform_moments_and_range():
    std = 0.02
    v = hash_uniform_f32(stream_key(1, 2), 0, 200_000, std).astype(np.float64)
    a = std * math.sqrt(3.0)
    assert v.min() >= -a and v.max() <= a
    assert abs(v.mean()) < 4 * std / math.sqrt(v.size)
    assert abs(v.std() - std) < 0.01 * std
    # the extremes of the 24-bit grid reach the ends of the interval
    assert v.max() > 0.999 * a and v.min() < -0.999 * a


def test_hash_slices_are_consistent():
    key = stream_key(3, 99)
    full = hash_u64(key, 0, 1000)
    assert np.array_equal(full[300:700], hash_u64(key, 300, 400))


def test_injection_frequency_matches_p():
    n = 20000
    for p in (0.0, 0.3, 0.7, 1.0):
        thr = inject_threshold(p)
        hits = sum(inject_draw(11, 0, pos, 1 + pos % 3) < thr for pos in range(n))
        if p in (0.0, 1.0):
            assert hits == int(p * n)
        else:
            sd = math.sqrt(n * p * (1 - p))
            assert abs(hits - p * n) < 5 * sd


def test_presets_parameter_counts():
    # The 31B-class workload is "~30.5B params"; a tied LM head gives 30.535B.
    assert abs(preset("31b").target_params() / 1e9 - 30.535) < 0.01
    # E2B-shaped target: 1.252B with a tied head.
    assert abs(preset("e2b").target_params() / 1e9 - 1.252) < 0.005
    t = preset("tiny")
    assert t.vocab == t.n_centroids * t.cluster_size


def test_inject_table_agrees_with_scalar_draws():
    from workloads import inject_table
    g = np.arange(100, 160, dtype=np.int64)
    g[:5] = -1
    tab = inject_table(g, 3, 0.6, 17, b=1).reshape(-1, 3)
    thr = inject_threshold(0.6)
    for pos in range(len(g)):
        for j in (1, 2, 3):
            want = g[pos] if (g[pos] >= 0 and inject_draw(17, 1, pos, j) < thr) else -1
            assert tab[pos, j - 1] == want
    full = inject_table(g, 2, 1.0, 3).reshape(-1, 2)
    assert np.array_equal(full[5:, 0], g[5:]) and np.all(full[:5] == -1)
    wrong = inject_table(g, 2, 0.0, 3, forced_wrong=True, vocab=150).reshape(-1, 2)
    assert np.array_equal(wrong[5:, 1], (g[5:] + 1) % 150)


def test_expert_stack_slices_equal_the_whole_tensor():
    from workloads import preset
    from workloads import synth as S
    from workloads.synth import ExpertStack
    for cfg in (preset("tiny-moe"), preset("tiny-moe", init="hash", dtype="bf16", seed=3)):
        E, Fe, d = cfg.n_experts, cfg.expert_ffn, cfg.d_model
        whole = S.gen_tensor(cfg, "exp_wd", 1, (E, d, Fe))
        st = ExpertStack(cfg, "exp_wd", 1, (E, d, Fe))
        for e in (0, 5, E - 1):
            assert np.array_equal(st[e], whole[e])
        assert len(st) == E


def test_q4_generator_codes_steps_and_slices():
    """4-bit tensors as drawn: codes are the top 4 bits of the tensor's stream, steps fp16 values
    on [2s/3, 4s/3) with s = std / sqrt(21.5), row slices equal the whole tensor's rows, and the
    weights (through the oracle's q4_weights) have about the configured standard deviation."""
    import oracle as O
    from workloads import synth as S
    from workloads.synth import ExpertStack
    cfg = preset("tiny-moe", init="hash", dtype="bf16", seed=3, weight_format="q4")
    q = S.gen_tensor(cfg, "wo", 0, (256, 512))
    assert q.codes.dtype == np.uint8 and q.codes.shape == (256, 512)
    assert q.steps.dtype == np.float16 and q.steps.shape == (256, 16)
    z = hash_u64(stream_key(cfg.seed, S.tensor_id("wo", 0)), 0, 10)
    assert q.codes.reshape(-1)[:10].tolist() == [int(v >> np.uint64(60)) for v in z]
    s = cfg.weight_std / math.sqrt(21.5)
    st = q.steps.astype(np.float64)
    assert st.min() >= 2 * s / 3 * (1 - 1e-3) and st.max() <= 4 * s / 3 * (1 + 1e-3)
    counts = np.bincount(q.codes.reshape(-1), minlength=16)
    assert counts.min() > 0.9 * q.codes.size / 16
    rows = S.gen_q4_rows(cfg, "wo", 0, 512, 37, 5)
    assert np.array_equal(rows.codes, q.codes[37:42]) and np.array_equal(rows.steps, q.steps[37:42])
    w = O.q4_weights(q.codes, q.steps)
    assert abs(w.std() / cfg.weight_std - 1) < 0.05
    E, Fe, d = cfg.n_experts, cfg.expert_ffn, cfg.d_model
    whole = S.gen_tensor(cfg, "exp_wd", 1, (E, d, Fe))
    st = ExpertStack(cfg, "exp_wd", 1, (E, d, Fe))
    for e in (0, 5, E - 1):
        assert np.array_equal(st[e].codes, whole.codes[e]) and np.array_equal(st[e].steps, whole.steps[e])
