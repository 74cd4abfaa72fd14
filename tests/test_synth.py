"""The seeded generators: determinism, bf16 exactness and workload shapes."""
import numpy as np

import synth


def test_streams_are_deterministic_and_independent():
    a = synth.normal(synth.stream(0, 2, 5), (4, 6))
    b = synth.normal(synth.stream(0, 2, 5), (4, 6))
    c = synth.normal(synth.stream(0, 2, 6), (4, 6))
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


def test_bf16_round_is_exact_and_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.1415926], dtype=np.float32)
    r = synth.bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0);
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6 -> 1 + 2^-6.
    np.testing.assert_array_equal(r[:4], np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], dtype=np.float32))
    assert (r.view(np.uint32) & 0xFFFF).max() == 0
    assert abs(float(r[4]) - 3.1415926) < 2 ** -7 * 2


def test_outlier_channels():
    rng = synth.stream(0, 2, 20)
    A = synth.outlier_activations(rng, 512, 2048, 0.01, 20.0)
    s = np.sqrt((A.astype(np.float64) ** 2).mean(axis=0))
    assert (s > 10).sum() == 20          # round(0.01 * 2048) outlier columns
    assert (A.view(np.uint32) & 0xFFFF).max() == 0


def test_workload_shapes_small():
    w = synth.WORKLOADS["xw-fp32-64x512"]
    A, B = synth.linear_operands(w, w.linears[0])
    assert A.shape == (64, 512) and B.shape == (512, 512) and A.dtype == np.float32
    assert np.std(B) * np.sqrt(512) == __import__("pytest").approx(1.0, rel=0.02)
    w2 = synth.WORKLOADS["llama3.2-1b-proj-2k"]
    down = [l for l in w2.linears if l.name == "down@0.5"][0]
    A2, B2 = synth.linear_operands(w2, down, m=64)
    assert A2.shape == (64, 8192) and B2.shape == (8192, 2048)
    Q, Kt, V = synth.attention_operands(synth.WORKLOADS["llama3.1-8b-layer-16k"], L=64)
    assert Q.shape == (64, 32, 128) and Kt.shape == (8, 128, 64) and V.shape == (64, 8, 128)


def test_row_prefix_is_stable_across_m():
    w = synth.WORKLOADS["llama3.1-8b-layer-16k"]
    lin = w.linears[0]
    a = synth.linear_activation(w, lin, m=40)
    b = synth.linear_activation(w, lin, m=13)
    np.testing.assert_array_equal(a[:13], b)


def test_int8_per_column_form():
    rng = np.random.default_rng(1)
    B = (rng.standard_normal((300, 40)) * rng.uniform(0.01, 3.0, size=40)).astype(np.float32)
    B[:, 7] = 0.0                                           # an all-zero column
    q, s = synth.int8_per_column(B)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (40,)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(q[:, 7] == 0) and s[7] == 1.0
    # each column's largest magnitude maps to +-127, and q * s is within half a step of B
    # (plus the float32 rounding of B / s, at most 127 * 2^-23 steps)
    cols = [c for c in range(40) if c != 7]
    assert np.all(np.abs(q[:, cols]).max(axis=0) == 127)
    assert np.all(np.abs(q.astype(np.float64) * s - B) <= (0.5 + 2e-5) * s.astype(np.float64))
