"""The seeded input generators: deterministic, rows nest, rows regenerate alone."""

import numpy as np

import synth


def test_activations_deterministic_and_nested():
    a = synth.activations_bf16(32, 5120, seed=0)
    b = synth.activations_bf16(32, 5120, seed=0)
    assert np.array_equal(a, b)
    a8 = synth.activations_bf16(8, 5120, seed=0)
    assert np.array_equal(a8, a[:8])
    assert not np.array_equal(synth.activations_bf16(8, 5120, seed=1), a8)


def test_outlier_columns():
    cols = synth.outlier_columns(5120)
    assert cols.size == 5 and len(set(cols.tolist())) == 5
    assert synth.outlier_columns(17408).size == 17
    assert synth.outlier_columns(256).size == 0
    x = synth.activations_f32(4, 5120, outliers=True)
    y = synth.activations_f32(4, 5120, outliers=False)
    assert np.array_equal(x[:, cols], y[:, cols] * np.float32(20))
    rest = np.setdiff1d(np.arange(5120), cols)
    assert np.array_equal(x[:, rest], y[:, rest])


def test_weight_rows_regenerate_alone():
    w = synth.weights_f32(600, 64, seed=0, stream="q0")
    rows = np.array([599, 0, 257, 256, 3])
    assert np.array_equal(synth.weights_f32(600, 64, seed=0, stream="q0", rows=rows), w[rows])
    assert abs(float(w.mean())) < 0.05 and abs(float(w.std()) - 1) < 0.05


def test_tiny_inputs():
    c = synth.tiny_codes(512, 256)
    s = synth.tiny_scale_values(512, 256)
    assert c.shape == (512, 128) and c.dtype == np.uint8
    assert s.shape == (512, 16) and s.min() >= 2.0 ** -4 and s.max() <= 4.0
    nib = np.concatenate([c & 0xF, c >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()
