"""Pins of the oracle's post-step passes that go beyond de-oscillation itself: Q-EMA
(TetraJet rebuttal, Question 4 and the overhead / hyperparameter answers) and the
de-oscillation step that also emits the next forward's Q_D(W)."""
import numpy as np

import oracle as O


def test_qema_beta_zero_is_the_weight():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((8, 64)).astype(np.float32)
    ema = rng.standard_normal((8, 64)).astype(np.float32)
    e, c, s = O.qema_step(w, ema, 0.0)
    assert np.array_equal(e.view(np.uint32), w.view(np.uint32))
    wc, ws = O.quantize(w, O.ROW, O.RNE)
    assert np.array_equal(c, wc) and np.array_equal(s, ws)


def test_qema_beta_one_keeps_the_average():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((4, 32)).astype(np.float32)
    ema = rng.standard_normal((4, 32)).astype(np.float32)
    e, _, _ = O.qema_step(w, ema, 1.0)
    assert np.array_equal(e.view(np.uint32), ema.view(np.uint32))


def test_qema_half_is_the_exact_midpoint():
    # beta = 1/2 on small integers: both products and their sum are exact in float32
    rng = np.random.default_rng(2)
    w = rng.integers(-1000, 1000, (4, 32)).astype(np.float32)
    ema = rng.integers(-1000, 1000, (4, 32)).astype(np.float32)
    e, _, _ = O.qema_step(w, ema, 0.5)
    assert np.array_equal(e.astype(np.float64), (w.astype(np.float64) + ema) / 2)


def test_qema_constant_weight_follows_the_geometric_closed_form():
    # ema_t = w + beta^t (ema_0 - w); float32 rounding adds at most ~2 ulp per step,
    # damped by beta, so |error| <= 2 * 2^-23 / (1 - beta) ~ 1.2e-4 at beta = 0.998
    beta = 0.998
    w = np.ones((1, 32), np.float32)
    ema = np.zeros((1, 32), np.float32)
    for t in range(1, 601):
        ema, _, _ = O.qema_step(w, ema, beta)
        if t in (1, 2, 10, 100, 600):
            want = 1.0 - np.float64(np.float32(beta)) ** t
            assert np.max(np.abs(ema.astype(np.float64) - want)) < 1.5e-4, t
    # one step from zero is (1 - beta) * w, not beta * w
    e1, _, _ = O.qema_step(w, np.zeros_like(w), beta)
    assert abs(float(e1[0, 0]) - 0.002) < 1e-6


def test_qema_is_a_convex_combination():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 64)) * np.exp2(rng.integers(-20, 20, (16, 1)))).astype(np.float32)
    ema = (w + rng.standard_normal((16, 64)).astype(np.float32) * 0.1).astype(np.float32)
    for beta in (0.9, 0.997, 0.998, 0.999):
        e, c, s = O.qema_step(w, ema, beta)
        lo = np.minimum(w, ema).astype(np.float64)
        hi = np.maximum(w, ema).astype(np.float64)
        slack = 2 * np.spacing(np.maximum(np.abs(lo), np.abs(hi)).astype(np.float32)).astype(np.float64)
        assert np.all(e >= lo - slack) and np.all(e <= hi + slack)
        wc, ws = O.quantize(e, O.ROW, O.RNE)
        assert np.array_equal(c, wc) and np.array_equal(s, ws)


def test_deosc_step_quantized_codes_survive_the_snap():
    """The fused pass may emit the codes it computes for w before the snap: snapping
    a flagged weight to its bin value keeps the block scale and the element's code.
    Checked on a window where many elements are flagged and snapped."""
    rng = np.random.default_rng(4)
    rows, cols = 64, 128
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w_prev, d_w, d_q = O.deosc_init(w)
    for step in range(12):
        # oscillate around bin edges: alternating steps of +-3e-4
        w = (w + np.float32(3e-4 * (1 if step % 2 == 0 else -1))).astype(np.float32)
        end = step == 11
        before = w.copy()
        out = O.deosc_step_quantized(w, w_prev, d_w, d_q, end, 4.0)
        w, w_prev, d_w, d_q, flags = out[:5]
        codes, scales = out[5:]
        if end:
            assert flags.sum() > 100
            assert not np.array_equal(w, before)
            bc, bs = O.quantize(before, O.ROW, O.RNE)
            assert np.array_equal(codes, bc) and np.array_equal(scales, bs)
        wc, ws = O.quantize(w, O.ROW, O.RNE)
        assert np.array_equal(codes, wc) and np.array_equal(scales, ws)
