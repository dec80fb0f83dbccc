"""Pins for the oracle's 4-bit block weights (q4_weights).

Source: page 5 "Gemma 4's MTP drafter explained: speculative decoding with llama.cpp", section
"Step 1 -- repackaging the QAT drafter": the QAT weights keep every 32-weight block of a weight
matrix on a 4-bit grid (at most 16 distinct values per block), which is Q4_0's own layout.
Reading of Q4_0 (the pages name it without spelling it out): per row, block j of 32 consecutive
weights has one fp16 step d_j and codes q in 0..15, weight = d_j * (q - 8).

The pins are special cases worked by hand, the page's structural property, the block index
(which columns a step moves) and a closed form of a row sum over structured codes."""

import numpy as np

import oracle as O


def test_codes_map_to_the_integers_minus_eight_to_seven():
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :]  # one block: 0..15 twice
    steps = np.array([[1.0]], dtype=np.float16)
    w = O.q4_weights(codes, steps)
    assert w.shape == (1, 32)
    assert w[0, :16].tolist() == [-8, -7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7]
    assert np.array_equal(w[0, 16:], w[0, :16])
    # code 8 is zero whatever the step
    z = O.q4_weights(np.full((3, 64), 8, np.uint8), np.full((3, 2), 3.5, np.float16))
    assert not z.any()


def test_step_is_the_fp16_value_and_products_are_exact():
    # fp16(0.1) = 0.0999755859375 exactly; 7 * that and -8 * that are exact in float64
    steps = np.array([[0.1, -2.5]], dtype=np.float16)
    codes = np.concatenate([np.full(32, 15, np.uint8), np.zeros(32, np.uint8)])[None, :]
    w = O.q4_weights(codes, steps)
    assert np.all(w[0, :32] == 7 * 0.0999755859375)
    assert np.all(w[0, 32:] == -8 * -2.5)


def test_each_block_has_at_most_16_values_on_its_step_grid():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (24, 256)).astype(np.uint8)
    steps = rng.uniform(1e-3, 1e-2, (24, 8)).astype(np.float16)
    w = O.q4_weights(codes, steps)
    for i in range(24):
        for j in range(8):
            blk = w[i, 32 * j:32 * j + 32]
            assert len(np.unique(blk)) <= 16
            m = blk / float(steps[i, j])
            assert np.array_equal(m, np.round(m)) and m.min() >= -8 and m.max() <= 7


def test_a_step_moves_exactly_its_own_block_of_its_own_row():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, (4, 128)).astype(np.uint8)
    codes[codes == 8] = 9  # no zero weights, so every scaled weight changes
    steps = np.full((4, 4), 0.5, np.float16)
    base = O.q4_weights(codes, steps)
    for i, j in ((0, 0), (2, 3), (3, 1)):
        s2 = steps.copy()
        s2[i, j] = 0.25
        diff = O.q4_weights(codes, s2) != base
        want = np.zeros_like(diff)
        want[i, 32 * j:32 * j + 32] = True
        assert np.array_equal(diff, want)


def test_row_sum_closed_form():
    # codes 0..15 twice in every block: the block's weights sum to d_j * (2*120 - 32*8) = -16 d_j
    K = 32 * 5
    codes = np.tile(np.arange(16, dtype=np.uint8), K // 16)[None, :].repeat(3, 0)
    steps = np.array([[0.5, 1.0, 2.0, 0.125, 4.0], [1, 1, 1, 1, 1], [3, -1, 0, 2, 0.25]],
                     dtype=np.float16)
    w = O.q4_weights(codes, steps)
    assert np.array_equal(w.sum(axis=1), -16.0 * steps.astype(np.float64).sum(axis=1))


def test_stacked_leading_axes_and_as_f64():
    from workloads import Q4Codes
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, (3, 16, 64)).astype(np.uint8)
    steps = rng.uniform(-1, 1, (3, 16, 2)).astype(np.float16)
    w = O.q4_weights(codes, steps)
    for e in range(3):
        assert np.array_equal(w[e], O.q4_weights(codes[e], steps[e]))
    tree = O.as_f64({"a": [Q4Codes(codes[0], steps[0])], "b": np.ones(3, np.float32)})
    assert np.array_equal(tree["a"][0], w[0]) and tree["b"].dtype == np.float64
